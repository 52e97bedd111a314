// Block quantizer of the KVarN method on gfx950.
//
// One workgroup (512 threads, 8 wave64) quantizes one 128-token x D-channel
// block of K or V (one layer, sequence, kv-head, chunk; D = 64, 128 or 256)
// at a time and walks the blocks of the launch persistently (stride = grid),
// loading the next block's bf16 input into registers while the current one
// is coded. Wave w owns tokens [16 w, 16 w + 16). NT = D / 16 is the number
// of 16-channel output tiles, KK = D / 32 the number of 32-channel input
// pieces.
//   1. load: lane (m = lane % 16, g = lane / 16) reads KK 16-byte pieces of
//      token 16 w + m (channels 32 kk + 8 g + [0, 8)), so one load instruction
//      covers 64 contiguous bytes of each of 16 rows; the pieces are the A
//      operands of the MFMAs;
//   2. Hadamard rotation along channels (rndamp article on KVarN, "How It
//      Works", item 1) as a dense product on the matrix cores:
//      y = x H_D with v_mfma_f32_16x16x32_bf16, KK x NT MFMAs per wave.
//      Sylvester's H_D has entry (-1)^popcount(i & j); split over the tile
//      indices, each 32 x 16 tile (kk, nt) of it is a sign
//      (-1)^popcount(kk & (nt/2)) times one of two lane-constant operands
//      (nt % 2), whatever D is. The result lands token by token: lane (n, g)
//      holds tokens 16 w + 4 g + r (r < 4) of channels 16 nt + n (nt < NT).
//      bf16 inputs and +-1 are exact and the products accumulate in fp32;
//      fp32 input is split exactly into three bf16 terms (three MFMAs per
//      product). With the rotation absorbed into the weights, the MFMAs run
//      on identity tiles (one per output tile), which copies x exactly;
//   3. dual-scaling normalization ("How It Works", item 2; abstract: both
//      axes of K and V): the squares P = y^2 stay in registers next to y.
//      Row step: each lane weighs its NT channels of each of its 4 tokens by
//      1/c^2 and the 16 lanes of a row combine their sums (two lane-pair
//      exchanges that halve the values, then two rotations), with no LDS and
//      no barrier. Column step: each lane weighs its 4 tokens of each of its
//      NT channels by 1/r^2, the four lane rows of the wave add up their
//      sums by two lane-swap steps (each halving the values a lane holds),
//      and the wave writes one partial per channel to LDS; after a barrier
//      wave w adds up channels (D/8) w + [0, D/8) only (512/D lanes per
//      channel, each taking D/64 of its 8 partials, the lanes meeting by DPP
//      adds), writes 1/c^2 to a shared D-entry array and, after a second
//      barrier, every lane reads the NT values of its channels. (Each wave
//      adding up all channels itself would need one barrier less but three
//      times the VALU instructions.)
//   4. per-token range step and 2-bit codes (v_cvt_pk_u8_f32): K codes of
//      four adjacent channels (four adjacent lanes) merge by a shift and
//      LDS OR atomics into a small per-wave staging area and leave
//      as D/16 contiguous bytes per lane (a wave writes its 16 token rows as
//      one 4D-byte span); V codes of a lane's 4 tokens form a byte in the
//      lane (shifts inside the bytes of words that each hold one token of
//      four channel tiles), and 4 x 4 byte transposes across the wave's rows
//      (two permlane swaps per pair of words) give each lane whole 4-byte
//      words of channel rows.
// The rotation is applied without its 1/sqrt(D) factor; that factor leaves
// the column scales and codes unchanged and is folded into the row scale.
// With D != 128 the row step's mean over D channels and the column step's
// mean over 128 tokens no longer cancel: the column step carries D/128 (an
// exact power of two here).
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

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr float kGrid = 1.9999980926513672f;  // 2 (1 - 2^-20)
constexpr float kTiny = 1.17549435e-38f;       // smallest normal fp32
// Global stores each wave issues per block after it prefetches the block
// after next into LDS (section 4: column scales, row scales, codes). The
// prefetch wait leaves all but one of them outstanding, so one store fewer
// than counted here (a compiler-merged or removed store) still waits for
// the prefetch; more stores only wait less long.
constexpr int kStoresAfterPrefetch = 3;
constexpr int kPrefetchLanded = waitcnt_vm(kStoresAfterPrefetch - 1);
static_assert(kStoresAfterPrefetch >= 2 && kStoresAfterPrefetch - 1 < 64, "prefetch wait count");

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// LDS. On gfx950 a ds_write_b32 is served one half-wave per pass with the
// dword address taken modulo 32 as its bank; a ds_read_b32 pair
// (ds_read2st64) of consecutive lanes reads consecutive dwords. The areas
// below are laid out for that model (for D = 128; the other head sizes use
// the same strides):
//  * cpart: the column step's partial sums, one per (wave u, channel c) at
//    cpart[CP_WAVE u + cp_index(c)], written by lane row g of the wave for
//    its channels [g D/4, (g + 1) D/4). Wave w adds up channels
//    (D/8) w + l / LPC (LPC = 512/D lanes each), lane l taking waves
//    (l % LPC) PPW + [0, PPW) (PPW = 8 / LPC). cp_index moves the D/4
//    channels of lane row g by 16 g words (D = 128, 256), so that the two
//    lane rows of a half-wave write distinct banks, and the wave strides
//    (72, 200, 312 words) put the 64 reading lanes of a wave on distinct
//    banks;
//  * ctot: the per-channel result of a column step (1/c^2, and 1/c after the
//    last one), written by the lanes that reduced the channel and read by
//    every lane for channels 16 nt + n (the four lane rows of a wave read the
//    same words);
//  * kst[wave]: K code staging, rows of KST_ROW = 4 NT + 4 words per group
//    of 4 tokens (word (token r, word k, quad q) at KST_ROW g + NT r + 4 k +
//    q; for D = 128 the 36-word rows put the two 16-lane rows of a half-wave
//    on disjoint banks);
//  * vst[buffer]: V code staging, word (channel j, wave w) at VST_ROW j + w
//    (9-word rows: the 32 channels of a half-wave's write fall on distinct
//    banks); two buffers alternated by V block, so that one barrier per
//    block orders the writes before the reads and the reads before the
//    buffer's next writes.
constexpr int VST_ROW = 9;

// Sizes of the kernel for head size DQ.
template <int DQ>
struct QDims {
  static_assert(DQ == 64 || DQ == 128 || DQ == 256, "head size");
  static constexpr int NT = DQ / 16;        // 16-channel output tiles
  static constexpr int KK = DQ / 32;        // 32-channel input pieces (MFMA steps)
  static constexpr int CPT = 4 * NT;        // values per lane: 4 tokens x NT channels
  static constexpr int LPC = 512 / DQ;      // lanes per channel in the column-step sum
  static constexpr int PPW = 8 / LPC;       // partial sums (waves) each of them adds
  static constexpr int CP_WAVE = DQ == 64 ? 72 : DQ == 128 ? 200 : 312;  // cpart wave stride
  static constexpr int KST_ROW = 4 * NT + 4;  // K staging words per group of 4 tokens
  static constexpr int CHUNK_CODE_BYTES = T * DQ / 4;
};
// cpart word of channel c within a wave's partials
template <int DQ>
__device__ __forceinline__ int cp_index(int c) {
  return DQ == 64 ? c : c + 16 * (c / (DQ / 4));
}
// Waves per SIMD the registers allow: three workgroups per CU for 64
// channels (at most 85 registers; 14% faster than two), two for 128, one
// for 256 (y and P alone take 128 registers there).
__host__ __device__ constexpr int quant_waves_per_simd(int dq) {
  return dq == 256 ? 2 : dq == 64 ? 6 : 4;
}

template <int DQ>
struct QuantSmem {
  alignas(16) float cpart[kWaves * QDims<DQ>::CP_WAVE];
  alignas(16) float ctot[DQ];
  alignas(16) uint32_t kst[kWaves][4 * QDims<DQ>::KST_ROW];
  alignas(16) uint32_t vst[2][DQ * VST_ROW];
  alignas(16) u32x4 hop[4][64];  // rotation operands of each lane (2, 3: negated)
  // bf16 input two blocks ahead, streamed by the wave straight into its own
  // slice (piece kk of lane l at xin[wave][kk][l], the order the direct
  // global-to-LDS load writes in)
  alignas(16) u32x4 xin[kWaves][QDims<DQ>::KK][64];
};

__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }
// 1 / max(x, smallest normal float) for x >= 0, the maximum taken on the bit
// patterns (non-negative floats order as their patterns do as unsigned
// integers), which needs no NaN canonicalization
__device__ __forceinline__ float rcp_floor(float x) {
  return __builtin_amdgcn_rcpf(__uint_as_float(max(__float_as_uint(x), __float_as_uint(kTiny))));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int kXor1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kXor2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kRor4 = 0x124;  // row_ror:4, lane i of a row reads lane (i + 4) % 16
constexpr int kRor8 = 0x128;  // row_ror:8

// kMax: maxima of non-negative values, taken on their bit patterns (the
// order of non-negative floats is that of their patterns as unsigned
// integers), which needs no NaN canonicalization and folds the DPP operand.
template <bool kMax>
__device__ __forceinline__ float combine(float a, float b) {
  if constexpr (kMax) return __uint_as_float(max(__float_as_uint(a), __float_as_uint(b)));
  else return a + b;
}

// Totals (kMax: maxima) over the 16 lanes of a row of four per-token values
// s[0..3]. Lane pairs 1 apart, then 2 apart, hand each other the values they
// do not keep, so that lane n is left with token tsel(n) = 2 (n % 2) +
// (n / 2) % 2 summed over its quad; rotations by 8 and by 4 lanes then add
// the four quads (lanes n, n + 4, n + 8, n + 12 hold the same token).
template <bool kMax>
__device__ __forceinline__ float row_reduce4(const float (&s)[4], int n) {
  const bool b0 = n & 1, b1 = n & 2;
  float k0 = b0 ? s[2] : s[0], k1 = b0 ? s[3] : s[1];
  const float e0 = b0 ? s[0] : s[2], e1 = b0 ? s[1] : s[3];
  k0 = combine<kMax>(k0, dpp_f<kXor1>(e0));
  k1 = combine<kMax>(k1, dpp_f<kXor1>(e1));
  float k = b1 ? k1 : k0;
  const float e = b1 ? k0 : k1;
  k = combine<kMax>(k, dpp_f<kXor2>(e));
  k = combine<kMax>(k, dpp_f<kRor8>(k));
  return combine<kMax>(k, dpp_f<kRor4>(k));
}
__device__ __forceinline__ int tsel(int n) { return 2 * (n & 1) + ((n >> 1) & 1); }
// Token R's value after row_reduce4, from the quad lane that holds it.
template <int R>
__device__ __forceinline__ float token_value(float x) {
  constexpr int l = 2 * (R & 1) + (R >> 1);
  return dpp_f<l * 0x55>(x);  // quad_perm [l, l, l, l]
}

// p[kOffset / 4] |= v on an LDS word, as a no-return LDS atomic. Written
// out because the compiler's form waits for every outstanding vector-memory
// operation first (it cannot tell the word from the LDS slice the input
// prefetch writes); the word is in the K staging area, which no prefetch
// touches. The wait for its completion is wave_lds_sync's lgkmcnt(0).
template <int kOffset>  // bytes
__device__ __forceinline__ void lds_or(uint32_t *p, uint32_t v) {
  static_assert(kOffset >= 0 && kOffset < 65536, "ds offset field");
  const uint32_t a = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint32_t *)p;
  asm volatile("ds_or_b32 %0, %1 offset:%2" ::"v"(a), "v"(v), "i"(kOffset) : "memory");
}

// K codes of the lane's token R, channel tiles 4 K + [0, 4), as the bytes of
// one word shifted to bit sh, ORed into staging word NT R + 4 K (for every R
// and K from the given ones on).
template <int DQ, int R, int K>
__device__ __forceinline__ void k_code_words(const float *y, const float (&qs)[4], uint32_t *base,
                                             int sh) {
  constexpr int NT = DQ / 16;
  uint32_t c = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    c = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(y[4 * (4 * K + i) + R], qs[R], 1.5f), i, c);
  lds_or<4 * (NT * R + 4 * K)>(base, c << sh);
  if constexpr (K + 1 < NT / 4)
    k_code_words<DQ, R, K + 1>(y, qs, base, sh);
  else if constexpr (R + 1 < 4)
    k_code_words<DQ, R + 1, 0>(y, qs, base, sh);
}

// LDS accesses of the wave complete and are visible to its other lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_s_waitcnt((0x7 << 4) | 0xF | (0x3 << 14));  // lgkmcnt(0) only
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ f32x4 mfma_bf16(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// B operand of the rotation for output-channel tile parity p. Lane (n, g),
// slot e multiplies input channel 32 kk + 8 g + e (slot e of the A operand's
// lane group g) into output channel 16 nt + n: popcount((32 kk + 8 g + e) &
// (16 nt + n)) splits into popcount(e & n), g bit 0 with n bit 3, g bit 1
// with nt bit 0 (= p), and kk & (nt / 2); the last part is the tile's sign,
// the others are fixed per lane and slot.
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
// 16 nt + n takes input channel 32 (nt / 2) + 8 g + e exactly when
// g = 2 (nt % 2) + n / 8 and e = n % 8.
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

// acc[nt] += x (input channels 32 kk + [0, 32) of the wave's 16 tokens) times
// tile (kk, nt) of the rotation (kk a constant after unrolling). A Hadamard
// tile with a negative sign takes the negated operand hp[2 + nt % 2] (kept in
// LDS next to the positive ones, so that no sign flips cost vector
// instructions); the identity has one tile per output tile, at kk = nt / 2.
template <bool kRotate, int NT>
__device__ __forceinline__ void rotate_step(f32x4 (&acc)[NT], const u32x4 &x, const u32x4 (&hp)[4],
                                            int kk) {
  if constexpr (kRotate) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const bool neg = __builtin_popcount((nt >> 1) & kk) & 1;
      acc[nt] = mfma_bf16(x, hp[(neg ? 2 : 0) + (nt & 1)], acc[nt]);
    }
  } else {
    acc[2 * kk] = mfma_bf16(x, hp[0], acc[2 * kk]);
    acc[2 * kk + 1] = mfma_bf16(x, hp[1], acc[2 * kk + 1]);
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

// bf16 input of block bi: a wave-uniform base (its first token row) plus the
// lane's fixed byte offset xlane = 2 ti st + 16 g (token ti, channels 8 g ..).
__device__ __forceinline__ const char *x_block_bf16(const QuantArgs &a, const BlockIdx &bi,
                                                    int64_t xlane) {
  return static_cast<const char *>(a.x) +
         2 * ((int64_t)bi.b * a.sb + (int64_t)bi.h * a.sh + (int64_t)(bi.kc * T) * a.st) + xlane;
}

// Piece kk of the lane's token row: channels 32 kk + 8 g + [0, 8).
template <int KK>
__device__ __forceinline__ void load_bf16_block(const QuantArgs &a, const BlockIdx &bi,
                                                int64_t xlane, u32x4 (&xr)[KK]) {
  const u32x4 *src = reinterpret_cast<const u32x4 *>(x_block_bf16(a, bi, xlane));
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) xr[kk] = __builtin_nontemporal_load(src + 4 * kk);
}

// The same pieces as load_bf16_block, copied by the memory system straight
// into the wave's LDS slice (global_load_lds_dwordx4: lane l's 16 bytes land
// at slice[kk][l]); counted by vmcnt like any load.
template <int KK>
__device__ __forceinline__ void prefetch_bf16_block_lds(const QuantArgs &a, const BlockIdx &bi,
                                                        int64_t xlane, u32x4 (*slice)[64]) {
  const u32x4 *src = reinterpret_cast<const u32x4 *>(x_block_bf16(a, bi, xlane));
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    __builtin_amdgcn_global_load_lds(src + 4 * kk,
                                     (__attribute__((address_space(3))) void *)&slice[kk][0], 16, 0, 0);
}

// b * 0x01010101 for b < 256: byte 0 of b in all four bytes, by a byte
// permute (a full-rate instruction; a 32-bit integer multiply issues at a
// quarter of the rate)
__device__ __forceinline__ uint32_t bytes4(uint32_t b) { return __builtin_amdgcn_perm(0u, b, 0u); }

// Pairwise sum of N values (N a power of two), halves first.
template <int N>
__device__ __forceinline__ float tree_sum(const float *q) {
  if constexpr (N == 1) {
    return q[0];
  } else {
    return tree_sum<N / 2>(q) + tree_sum<N / 2>(q + N / 2);
  }
}

// V codes: lane g of the four rows (lanes 16 apart) holds words p0, p1 whose
// byte j is the V byte of channel 16 j + n (16 (4 + j) + n) for byte column g.
// Two 4 x 4 byte transposes across the rows: lane g ends with the words of
// channels 16 g + n (o0) and 64 + 16 g + n (o1), byte g' from row g'. Rows g
// and g ^ 2 (permlane32) trade the column pair the other keeps, then rows g
// and g ^ 1 (permlane16) the column the other keeps.
__device__ __forceinline__ void v_transpose(uint32_t p0, uint32_t p1, int t, uint32_t &o0,
                                            uint32_t &o1) {
  const uint32_t hi = (t >> 5) & 1, odd = (t >> 4) & 1;  // g / 2, g % 2
  const uint32_t k1 = __builtin_amdgcn_perm(p1, p0, 0x05040100u + bytes4(2u * hi));
  const uint32_t s1 = __builtin_amdgcn_perm(p1, p0, 0x07060302u - bytes4(2u * hi));
  const auto x1 = __builtin_amdgcn_permlane32_swap(s1, s1, false, false);
  const uint32_t r1 = hi ? x1[0] : x1[1];
  const uint32_t k2 = __builtin_amdgcn_perm(r1, k1, 0x06040200u + bytes4(odd));
  const uint32_t s2 = __builtin_amdgcn_perm(r1, k1, 0x07050301u - bytes4(odd));
  const auto x2 = __builtin_amdgcn_permlane16_swap(s2, s2, false, false);
  const uint32_t r2 = odd ? x2[0] : x2[1];
  // byte rho of the word is row rho's byte: kept (rho = g: byte 0,
  // rho = g ^ 2: byte 2) or received (rho = g ^ 1: byte 4, g ^ 3: byte 6),
  // i.e. byte f(rho ^ g) with f = (0, 4, 2, 6)
  const uint32_t sel =
      __builtin_amdgcn_perm(0u, 0x06020400u, 0x03020100u ^ bytes4((uint32_t)((t >> 4) & 3)));
  o0 = __builtin_amdgcn_perm(r2, k2, sel);
  o1 = __builtin_amdgcn_perm(r2, k2, sel + 0x01010101u);
}

// kRotate = false: the input is already rotated (rotation absorbed into the
// model's weights) and the MFMAs copy it through identity tiles.
// kPositions: x is a one-chunk window per (b, h); block (b, h) re-quantizes
// cache chunk pos[b] / 128 only when pos[b] % 128 == 127, i.e. when the token
// just appended at pos[b] filled its chunk (kvarn_append_rebalance).
template <int DQ, bool kF32, bool kRotate, bool kPositions>
__global__ __launch_bounds__(kThreads, quant_waves_per_simd(DQ)) void quantize_block_kernel(
    QuantArgs a) {
  using Q = QDims<DQ>;
  constexpr int NT = Q::NT, KK = Q::KK, CPT = Q::CPT, LPC = Q::LPC, PPW = Q::PPW;
  __shared__ QuantSmem<DQ> sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar LDS addresses
  const int n = lane & 15, g = lane >> 4;
  const int ti = 16 * wv + n;  // token whose input row the lane loads
  const int64_t xlane = 2 * (int64_t)ti * a.st + 16 * g;  // its bytes within a bf16 block
  const int64_t nch = a.capacity / T;
  // the channel whose column-step sum this lane takes part in
  const int ch = (DQ / 8) * wv + lane / LPC;
  // r' from the running maximum: the unscaled rotation's 1/sqrt(D) and the
  // 1/2 of the range step, or the 1/2 alone for pre-rotated input
  const float range_factor = kRotate ? range_from_unscaled(DQ) : kRangeFromRotated;

  // Positions mode runs after every append, and a chunk closes on one step in
  // 128: a workgroup none of whose blocks closes leaves before it loads
  // anything (the loop below skips the non-closing blocks of the others).
  if constexpr (kPositions) {
    bool any = false;
    for (uint32_t b0 = blockIdx.x; b0 < a.nblocks; b0 += gridDim.x) {
      const int pos = a.pos[split_block(a, b0).b];
      any |= pos >= 0 && pos < a.capacity && pos % T == T - 1;
    }
    if (!any) return;  // uniform over the workgroup
  }

  // the lane's two rotation operands live in LDS (registers are held by y,
  // P and the next block's input through the balancing)
  if (tid < 64) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const u32x4 h = kRotate ? hadamard_operand(lane, p) : identity_operand(lane, p);
      sm.hop[p][lane] = h;
      sm.hop[2 + p][lane] = h ^ 0x80008000u;  // bf16 sign bits flipped
    }
  }
  lds_barrier();

  // bf16 input: the block being started is in xn (registers); the next one
  // is in the wave's LDS slice xin[wv] or on its way there
  u32x4 xn[KK];
  uint32_t blk = blockIdx.x;
  if constexpr (!kF32) {
    if (blk < a.nblocks) {
      load_bf16_block<KK>(a, split_block(a, blk), xlane, xn);
      prefetch_bf16_block_lds<KK>(a, split_block(a, min(blk + gridDim.x, a.nblocks - 1)), xlane,
                                  sm.xin[wv]);
    }
    // waited for here once, so that the loop head does not merge the first
    // loads into every block's wait
    __builtin_amdgcn_s_waitcnt(kVmcntZero);
  }
  auto rotate_f32 = [&](const BlockIdx &bi, f32x4 (&acc)[NT]) {  // three bf16 terms per piece
    const u32x4 hp[4] = {sm.hop[0][lane], sm.hop[1][lane], sm.hop[2][lane], sm.hop[3][lane]};
    const f32x4 *src =
        reinterpret_cast<const f32x4 *>(static_cast<const float *>(a.x) + x_offset(a, bi, ti)) +
        2 * g;
    f32x4 xv[2 * KK];
#pragma unroll
    for (int q = 0; q < 2 * KK; ++q) xv[q] = __builtin_nontemporal_load(src + 8 * (q >> 1) + (q & 1));
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      u32x4 th, tm, tl;
      split_bf16x3(xv[2 * kk], xv[2 * kk + 1], th, tm, tl);
      rotate_step<kRotate, NT>(acc, tl, hp, kk);
      rotate_step<kRotate, NT>(acc, tm, hp, kk);
      rotate_step<kRotate, NT>(acc, th, hp, kk);
    }
  };
  auto rotate_bf16 = [&](const u32x4 (&x)[KK], f32x4 (&acc)[NT]) {
    const u32x4 hp[4] = {sm.hop[0][lane], sm.hop[1][lane], sm.hop[2][lane], sm.hop[3][lane]};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) rotate_step<kRotate, NT>(acc, x[kk], hp, kk);
  };

  int vbuf = 0;  // V staging buffer of the next V block
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
    // y[4 nt + r]: token 16 wv + 4 g + r, channel 16 nt + n
    float y[CPT], p[CPT];
    f32x4 gram = {0.f, 0.f, 0.f, 0.f};  // bf16: x x^T of the wave's 16 tokens
    {
      f32x4 acc[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (kF32) {
        rotate_f32(bi, acc);
      } else {
        rotate_bf16(xn, acc);
        // first row step by Parseval: sum_j y_j^2 = D sum_k x_k^2 (1 sum_k
        // x_k^2 without the rotation); the diagonal of x x^T, from the same
        // operand registers, lands in lane (n, g = n / 4), register n % 4
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) gram = mfma_bf16(xn[kk], xn[kk], gram);
        // next block's input from the LDS slice into xn, then the block after
        // it into the slice: in flight during this whole block and the next
        // one's rotation (the LDS-only barriers below do not wait for it).
        // The slice's load was issued one block ago and was followed by that
        // block's kStoresAfterPrefetch stores (a skipped block waits for
        // everything instead); vector-memory operations retire in order, so
        // kPrefetchLanded means the load has landed while the last block's
        // stores may still be in flight. The slice is the wave's own: LDS
        // ordering within the wave is all that is needed after that.
        __builtin_amdgcn_s_waitcnt(kPrefetchLanded);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) xn[kk] = sm.xin[wv][kk][lane];
        __builtin_amdgcn_s_waitcnt((0x7 << 4) | 0xF | (0x3 << 14));  // lgkmcnt(0): reads done
        const uint32_t nb = min(blk + 2 * gridDim.x, a.nblocks - 1);
        prefetch_bf16_block_lds<KK>(a, split_block(a, nb), xlane, sm.xin[wv]);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        y[4 * nt + 0] = acc[nt].x; y[4 * nt + 1] = acc[nt].y;
        y[4 * nt + 2] = acc[nt].z; y[4 * nt + 3] = acc[nt].w;
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
    // Wave priorities: the sweeps are a chain of short sections between
    // workgroup barriers, and a barrier waits for the workgroup's slowest
    // wave, while the other resident workgroup's rotation and code packing
    // is work without such a chain. The sweeps' FMA chains run at priority
    // 2, the reductions that lead into and out of the barriers (the first
    // row step, the column step after its barrier, the row step's lane
    // reduction) at 3, and rotation and codes at 0, where they fill the
    // issue slots the sweeps leave (about 10% less time per launch than
    // equal priorities).
    float w[NT];     // 1/c^2 of channels 16 nt + n; 1/c after the last column step
    float cm = 1.f;  // c^2 of channel ch after a column step, then c
    __builtin_amdgcn_s_setprio(3);
    if (a.iters > 0) {
      // v_i = 1 / (D r_i^2) of the lane's tokens: v_i = 1 / sum_j P_ij / c_j^2,
      // and the column step's c_j^2 = (1/T) sum_i P_ij / r_i^2 is
      // (D/T) sum_i P_ij v_i (D/T = 1 for the square block). A zero row or
      // column (all its P are 0) takes the reciprocal of the smallest normal
      // number instead of 1: its products are 0 either way, and its stored
      // scales are set below.
      float v[4];
      {
        // first row step (c = 1): v_i = 1 / sum_j P_ij
        float tot;
        if constexpr (kF32) {
          float s[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float q[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) q[nt] = p[4 * nt + r];
            s[r] = tree_sum<NT>(q);
          }
          tot = row_reduce4<false>(s, n);
        } else {
          // token 4 g + tsel(n) sits in lane 16 g + 4 g + tsel(n), register tsel(n)
          const int r = n & 3;
          const float d = (r & 2) ? ((r & 1) ? gram.w : gram.z) : ((r & 1) ? gram.y : gram.x);
          const int t = tid;
          const int src = 20 * ((t >> 4) & 3) + tsel(t);
          tot = (kRotate ? (float)DQ : 1.f) * __shfl(d, src, 64);
        }
        const float vt = rcp_floor(tot);
        v[0] = token_value<0>(vt); v[1] = token_value<1>(vt);
        v[2] = token_value<2>(vt); v[3] = token_value<3>(vt);
      }
      for (int it = 0;;) {
        __builtin_amdgcn_s_setprio(2);
        // column step: the lane's NT partial sums (its 4 tokens of channels
        // 16 nt + n), added up over the wave's four lane rows, go to LDS;
        // the LPC lanes of channel ch then add up its 8 partials (one per
        // wave), PPW each, and meet by DPP adds
        float cp[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          cp[nt] = fmaf(p[4 * nt + 3], v[3],
                        fmaf(p[4 * nt + 2], v[2], fmaf(p[4 * nt + 1], v[1], p[4 * nt] * v[0])));
        {
          // rows g and g ^ 2 (half-wave swap), then g and g ^ 1 (row swap):
          // each swap hands over the half of the values the lane does not
          // keep, so lane row g is left with channels 16 (g NT/4 + k) + n,
          // k < NT/4, summed over the wave's 16 tokens
          constexpr int NH = NT / 2, NQ = NT / 4;
          float h[NH];
#pragma unroll
          for (int j = 0; j < NH; ++j) {
            const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(cp[j]),
                                                            __float_as_uint(cp[j + NH]), false, false);
            h[j] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
          }
          float *pw = sm.cpart + Q::CP_WAVE * wv;
#pragma unroll
          for (int k = 0; k < NQ; ++k) {
            const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(h[k]),
                                                            __float_as_uint(h[k + NQ]), false, false);
            pw[cp_index<DQ>(16 * (g * NQ + k) + n)] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
          }
        }
        lds_barrier();
        __builtin_amdgcn_s_setprio(3);
        {
          const float *pr = sm.cpart + Q::CP_WAVE * ((lane % LPC) * PPW) + cp_index<DQ>(ch);
          float q[PPW];
#pragma unroll
          for (int i = 0; i < PPW; ++i) q[i] = pr[Q::CP_WAVE * i];  // wave (lane % LPC) PPW + i
          cm = tree_sum<PPW>(q);
          cm += dpp_f<kXor1>(cm);
          if constexpr (LPC >= 4) cm += dpp_f<kXor2>(cm);
          if constexpr (LPC >= 8) cm += lane_xor<4>(cm);
          if constexpr (DQ != T) cm *= (float)DQ / (float)T;  // a power of two
        }
        if (++it == a.iters) break;
        // 1/c^2 of channel ch (its LPC lanes write the same value), then
        // every lane takes channels 16 nt + n
        sm.ctot[ch] = rcp_floor(cm);
        lds_barrier();
        {
          const float *pg = sm.ctot + n;
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) w[nt] = pg[16 * nt];
        }
        __builtin_amdgcn_s_setprio(2);
        // row step: r_i^2 = (1/D) sum_j P_ij / c_j^2  ->  v_i = 1 / sum_j P_ij / c_j^2
        float s[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float e = p[r] * w[0];
#pragma unroll
          for (int nt = 1; nt < NT; ++nt) e = fmaf(p[4 * nt + r], w[nt], e);
          s[r] = e;
        }
        __builtin_amdgcn_s_setprio(3);
        const float tot = row_reduce4<false>(s, n);
        const float vt = rcp_floor(tot);
        v[0] = token_value<0>(vt); v[1] = token_value<1>(vt);
        v[2] = token_value<2>(vt); v[3] = token_value<3>(vt);
      }
      // c and 1/c of channel ch (a zero column keeps c = 1)
      const float ic = cm > 0.f ? __builtin_amdgcn_rsqf(cm) : 1.f;
      cm = cm > 0.f ? cm * ic : 1.f;  // c = c^2 / sqrt(c^2)
      sm.ctot[ch] = ic;
      lds_barrier();
      {
        const float *pg = sm.ctot + (tid & 15);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) w[nt] = pg[16 * nt];
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) w[nt] = 1.f;
    }

    __builtin_amdgcn_s_setprio(0);
    // ---- 4. range step and codes --------------------------------------------
    // The three global stores below (column scales, row scales, codes) are
    // issued by every wave of every block that is not skipped, each with
    // active lanes in every wave: they are the kStoresAfterPrefetch that the
    // prefetch wait counts on.
    if (lane % LPC == 0)  // store 1 of 3; wave wv holds the column scales of channels (D/8) wv + [0, D/8)
      a.col_scale[(bh * nch + chunk) * DQ + ch] = cm;
    float mx[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        y[4 * nt + r] *= w[nt];
        mx[r] = fmaxf(mx[r], fabsf(y[4 * nt + r]));
      }
    const float m = row_reduce4<true>(mx, n);  // token 4 g + tsel(n)
    if (n < 4) {  // store 2 of 3; lane t % 16 < 4 of row (t / 16) % 4: token 4 (t / 16) + tsel(t)
      const int t = tid;
      a.row_scale[bh * a.capacity + (int64_t)chunk * T + 4 * (t >> 4) + tsel(t)] = m * range_factor;
    }
    const float qt = m > 0.f ? kGrid * rcp(m) : 0.f;
    const float qs[4] = {token_value<0>(qt), token_value<1>(qt), token_value<2>(qt),
                         token_value<3>(qt)};

    uint8_t *cbase = a.codes + (bh * nch + chunk) * Q::CHUNK_CODE_BYTES;
    if (a.kind == KVARN_K) {
      // word (r, k) of a lane: byte i = code of token 4 g + r, channel
      // 16 (4 k + i) + n; shifted to bit 2 (n % 4) and ORed over the quad it
      // becomes token-row byte 16 k + 4 i + n / 4 (channels 4 (4 k + i) +
      // n / 4 .. + 4). The ORs are LDS atomics into the staging words, which
      // the row's lanes clear first (a wave's LDS operations complete in
      // order).
      const int t = tid;
      const int s = t & 3, q = (t >> 2) & 3;
      uint32_t *ks = &sm.kst[wv][0] + Q::KST_ROW * ((t >> 4) & 3);
      if constexpr (NT == 4) {
        ks[n] = 0u;
      } else if constexpr (NT == 8) {
        *reinterpret_cast<u32x2 *>(ks + 2 * n) = u32x2{0u, 0u};
      } else {
        *reinterpret_cast<u32x4 *>(ks + 4 * n) = u32x4{0u, 0u, 0u, 0u};
      }
      k_code_words<DQ, 0, 0>(y, qs, ks + q, 2 * (tid & 3));
      wave_lds_sync();
      // lane n stores bytes [NT s, NT s + NT) of the row of token 4 g + q:
      // token-row bytes 16 k + 4 i + q' (quad q'), gathered from the four
      // quads' words of (token q, word k); the wave's 16 token rows are one
      // contiguous span, of which the lane's bytes start at (D/16) (t % 512)
      if constexpr (DQ == 64) {  // k = 0, byte i = s of each word
        const u32x4 wq = *reinterpret_cast<const u32x4 *>(ks + 4 * q);
        const uint32_t sel = 0x0C0C0400u + 0x0101u * (uint32_t)s;  // bytes s, 4 + s, zero, zero
        const uint32_t t01 = __builtin_amdgcn_perm(wq.y, wq.x, sel);
        const uint32_t t23 = __builtin_amdgcn_perm(wq.w, wq.z, sel);
        *reinterpret_cast<uint32_t *>(cbase + 4 * (t & 511)) =
            __builtin_amdgcn_perm(t23, t01, 0x05040100u);  // store 3 of 3 (K)
      } else if constexpr (DQ == 128) {  // k = s / 2, bytes i = 2 (s % 2) + [0, 2)
        const u32x4 wq = *reinterpret_cast<const u32x4 *>(ks + 8 * q + 4 * (s >> 1));
        const uint32_t sel = 0x05010400u + bytes4(2u * (uint32_t)(s & 1));
        const uint32_t t01 = __builtin_amdgcn_perm(wq.y, wq.x, sel);
        const uint32_t t23 = __builtin_amdgcn_perm(wq.w, wq.z, sel);
        const u32x2 pk = {__builtin_amdgcn_perm(t23, t01, 0x05040100u),
                          __builtin_amdgcn_perm(t23, t01, 0x07060302u)};
        *reinterpret_cast<u32x2 *>(cbase + 8 * (t & 511)) = pk;  // store 3 of 3 (K)
      } else {  // k = s, all four bytes of each word: a 4 x 4 byte transpose
        const u32x4 wq = *reinterpret_cast<const u32x4 *>(ks + 16 * q + 4 * s);
        const uint32_t a01 = __builtin_amdgcn_perm(wq.y, wq.x, 0x05010400u);  // x0 y0 x1 y1
        const uint32_t b01 = __builtin_amdgcn_perm(wq.y, wq.x, 0x07030602u);  // x2 y2 x3 y3
        const uint32_t a23 = __builtin_amdgcn_perm(wq.w, wq.z, 0x05010400u);
        const uint32_t b23 = __builtin_amdgcn_perm(wq.w, wq.z, 0x07030602u);
        const u32x4 pk = {__builtin_amdgcn_perm(a23, a01, 0x05040100u),
                          __builtin_amdgcn_perm(a23, a01, 0x07060302u),
                          __builtin_amdgcn_perm(b23, b01, 0x05040100u),
                          __builtin_amdgcn_perm(b23, b01, 0x07060302u)};
        *reinterpret_cast<u32x4 *>(cbase + 16 * (t & 511)) = pk;  // store 3 of 3 (K)
      }
    } else {
      // Byte j of pw[m] is the V byte of channel 16 (4 m + j) + n, tokens
      // 16 wv + 4 g + [0, 4) (byte column 4 wv + g of the channel row). The
      // codes of token r of four tiles are converted into the bytes of one
      // word, and the four tokens' words meet by shifts of 2 r within the
      // bytes (no field reaches the next byte).
      uint32_t pw[NT / 4];
#pragma unroll
      for (int m4 = 0; m4 < NT / 4; ++m4) {
        uint32_t xr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          xr[r] = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            xr[r] = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(y[4 * (4 * m4 + j) + r], qs[r], 1.5f), j,
                                                   xr[r]);
        }
        pw[m4] = (xr[0] | (xr[1] << 2)) | ((xr[2] << 4) | (xr[3] << 6));
      }
      // lane g ends with the words of channels 16 g + n + 64 m (byte column
      // 4 wv + [0, 4)), which go through LDS so that the block leaves as
      // contiguous stores of D/16 bytes per thread
      const int t = tid;
      uint32_t *vs = &sm.vst[vbuf][0];
      if constexpr (DQ == 64) {
        uint32_t o0, o1;
        v_transpose(pw[0], pw[0], t, o0, o1);  // the second word is unused
        vs[VST_ROW * (t & 63) + (t >> 6)] = o0;
      } else {
#pragma unroll
        for (int m2 = 0; m2 < NT / 8; ++m2) {
          uint32_t o0, o1;
          v_transpose(pw[2 * m2], pw[2 * m2 + 1], t, o0, o1);
          vs[VST_ROW * ((t & 63) + 128 * m2) + (t >> 6)] = o0;
          vs[VST_ROW * ((t & 63) + 128 * m2 + 64) + (t >> 6)] = o1;
        }
      }
      vbuf ^= 1;
      lds_barrier();
      // the channel row j (32 bytes: the words of waves 0..7) starts at 32 j;
      // thread u stores bytes [(D/16) u, (D/16) (u + 1)) of the block's V codes
      const int u = tid;
      if constexpr (DQ == 64) {  // channel u / 8, word of wave u % 8
        *reinterpret_cast<uint32_t *>(cbase + 4 * u) = vs[VST_ROW * (u >> 3) + (u & 7)];  // store 3 of 3 (V)
      } else if constexpr (DQ == 128) {  // channel u / 4, words of waves 2 (u % 4) + [0, 2)
        const uint32_t *src = vs + VST_ROW * (u >> 2) + 2 * (u & 3);
        const u32x2 word = {src[0], src[1]};
        *reinterpret_cast<u32x2 *>(cbase + 8 * u) = word;  // store 3 of 3 (V)
      } else {  // channel u / 2, words of waves 4 (u % 2) + [0, 4)
        const uint32_t *src = vs + VST_ROW * (u >> 1) + 4 * (u & 1);
        const u32x4 word = {src[0], src[1], src[2], src[3]};
        *reinterpret_cast<u32x4 *>(cbase + 16 * u) = word;  // store 3 of 3 (V)
      }
    }
  }
  // the last prefetch into the LDS slice lands before the workgroup (and its
  // LDS) goes away
  if constexpr (!kF32) __builtin_amdgcn_s_waitcnt(kVmcntZero);
}

}  // namespace

template <int DQ>
static hipError_t launch_quantize_dq(const QuantArgs &a, hipStream_t s) {
  // resident workgroups per CU as the registers allow (quant_waves_per_simd
  // x 4 SIMDs / 8 waves); each walks blocks strided by the grid
  const uint32_t resident = (uint32_t)(quant_waves_per_simd(DQ) / 2) * (uint32_t)device_cus();
  const uint32_t blocks = a.nblocks < resident ? a.nblocks : resident;
  const bool rot = !(a.flags & KVARN_FLAG_NO_ROTATE);
#define KVARN_LAUNCH_QUANT(F32, ROT, POS)                                                   \
  hipLaunchKernelGGL((quantize_block_kernel<DQ, F32, ROT, POS>), dim3(blocks), dim3(kThreads), 0, \
                     s, a)
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

hipError_t launch_quantize(const QuantArgs &a, hipStream_t s) {
  if (a.nblocks == 0) return hipSuccess;
  switch (a.head_dim) {
    case 64: return launch_quantize_dq<64>(a, s);
    case 256: return launch_quantize_dq<256>(a, s);
    default: return launch_quantize_dq<128>(a, s);
  }
}

}  // namespace kvarn
