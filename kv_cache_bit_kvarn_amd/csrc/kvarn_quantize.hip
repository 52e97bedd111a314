// Block quantizer of the KVarN method on gfx950.
//
// One workgroup (512 threads, 8 wave64) quantizes one 128-token x 128-channel
// block of K or V (one layer, sequence, kv-head, chunk) at a time and walks
// the blocks of the launch persistently (stride = grid), loading the next
// block's bf16 input into registers while the current one is coded. Wave w
// owns tokens [16 w, 16 w + 16).
//   1. load: lane (m = lane % 16, g = lane / 16) reads four 16-byte pieces of
//      token 16 w + m (channels 32 kk + 8 g + [0, 8)), so one load instruction
//      covers 64 contiguous bytes of each of 16 rows; the pieces are the A
//      operands of the MFMAs;
//   2. Hadamard rotation along channels (rndamp article on KVarN, "How It
//      Works", item 1) as a dense product on the matrix cores:
//      y = x H_128 with v_mfma_f32_16x16x32_bf16, 32 MFMAs per wave.
//      Sylvester's H_128 has entry (-1)^popcount(i & j); split over the tile
//      indices, each 32 x 16 tile (kk, nt) of it is a sign
//      (-1)^popcount(kk & (nt/2)) times one of two lane-constant operands
//      (nt % 2), the sign going onto the input piece. The result lands token
//      by token: lane (n, g) holds tokens 16 w + 4 g + r (r < 4) of channels
//      16 nt + n (nt < 8). bf16 inputs and +-1 are exact and the products
//      accumulate in fp32; fp32 input is split exactly into three bf16 terms
//      (three MFMAs per product). With the rotation absorbed into the
//      weights, the MFMAs run on identity tiles (one per output tile), which
//      copies x exactly;
//   3. dual-scaling normalization ("How It Works", item 2; abstract: both
//      axes of K and V): the squares P = y^2 stay in registers next to y.
//      Row step: each lane weighs its 8 channels of each of its 4 tokens by
//      1/c^2 (8 registers) and the 16 lanes of a row combine their sums
//      (two lane-pair exchanges that halve the values, then two rotations),
//      with no LDS and no barrier. Column step: each lane weighs its 4 tokens
//      of each of its 8 channels by 1/r^2 and writes the 8 partial sums to
//      LDS unreduced; after a barrier wave w adds up channels 16 w + [0, 16)
//      only (lane l: channel 16 w + l / 4, 8 of its 32 partials, the quad's
//      four lanes meeting by DPP adds), writes 1/c^2 to a shared 128-entry
//      array and, after a second barrier, every lane reads the 8 values of
//      its channels. (Each wave adding up all 128 channels itself would need
//      one barrier less but three times the VALU instructions.)
//   4. per-token range step and 2-bit codes (v_cvt_pk_u8_f32): K codes of
//      four adjacent channels (four adjacent lanes) merge by a shift and an
//      OR across the quad, pass through a small per-wave LDS area and leave
//      as 8 contiguous bytes per lane (a wave writes its 16 token rows as
//      one 512-byte span); V codes of a lane's 4 tokens form a byte in the
//      lane (shifts inside the bytes of words that each hold one token of
//      four channel tiles), and a 4 x 4 byte transpose across the wave's rows
//      (two permlane swaps) gives each lane two whole 4-byte words of channel
//      rows.
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

namespace {

constexpr int kThreads = 512;
constexpr int kWaves = kThreads / 64;
constexpr int CPT = 32;                        // values per lane: 4 tokens x 8 channels
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
// below are laid out for that model:
//  * cpart: the column step's partial sums, cp[nt] of lane l of wave u at
//    cpart[CP_PLANE nt + CP_WAVE u + l]. A wave's write of one nt covers 64
//    consecutive words; reading lane l of wave w takes plane w, channel
//    16 w + l / 4 of waves 2 (l % 4) + s (s < 2) and rows r, at
//    CP_PLANE w + CP_WAVE (2 (l % 4) + s) + 16 r + l / 4, and the 72-word
//    wave stride puts the four lanes of a quad 144 words (16 banks) apart, so
//    neither side has bank conflicts;
//  * ctot: the per-channel result of a column step (1/c^2, and 1/c after the
//    last one), written by the wave that reduced the channel and read by
//    every lane for channels 16 nt + n (the four lane rows of a wave read the
//    same words);
//  * kst[wave]: K code staging, rows of KST_ROW words per group of 4 tokens
//    (word (token r, half k, quad q) at KST_ROW g + 8 r + 4 k + q; the
//    36-word rows put the two 16-lane rows of a half-wave on disjoint
//    banks);
//  * vst[buffer]: V code staging, word (channel j, wave w) at VST_ROW j + w
//    (9-word rows: the 32 channels of a half-wave's write fall on distinct
//    banks); two buffers alternated by V block, so that one barrier per
//    block orders the writes before the reads and the reads before the
//    buffer's next writes.
constexpr int KST_ROW = 36;
constexpr int VST_ROW = 9;
constexpr int CP_WAVE = 72;
constexpr int CP_PLANE = kWaves * CP_WAVE;
struct QuantSmem {
  alignas(16) float cpart[8 * CP_PLANE];
  alignas(16) float ctot[D];
  alignas(16) uint32_t kst[kWaves][4 * KST_ROW];
  alignas(16) uint32_t vst[2][D * VST_ROW];
  alignas(16) u32x4 hop[4][64];  // rotation operands of each lane (2, 3: negated)
  // bf16 input two blocks ahead, streamed by the wave straight into its own
  // slice (piece kk of lane l at xin[wave][kk][l], the order the direct
  // global-to-LDS load writes in)
  alignas(16) u32x4 xin[kWaves][4][64];
};

__device__ __forceinline__ float rcp(float x) { return __builtin_amdgcn_rcpf(x); }

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
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
// tile (kk, nt) of the rotation. A Hadamard tile with a negative sign takes
// the negated operand hp[2 + nt % 2] (kept in LDS next to the positive ones,
// so that no sign flips cost vector instructions); the identity has one tile
// per output tile, at kk = nt / 2.
template <bool kRotate, int KK>
__device__ __forceinline__ void rotate_step(f32x4 (&acc)[8], const u32x4 &x, const u32x4 (&hp)[4]) {
  if constexpr (kRotate) {
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      const bool neg = __builtin_popcount((nt >> 1) & KK) & 1;
      acc[nt] = mfma_bf16(x, hp[(neg ? 2 : 0) + (nt & 1)], acc[nt]);
    }
  } else {
    acc[2 * KK] = mfma_bf16(x, hp[0], acc[2 * KK]);
    acc[2 * KK + 1] = mfma_bf16(x, hp[1], acc[2 * KK + 1]);
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
__device__ __forceinline__ void load_bf16_block(const QuantArgs &a, const BlockIdx &bi,
                                                int64_t xlane, u32x4 (&xr)[4]) {
  const u32x4 *src = reinterpret_cast<const u32x4 *>(x_block_bf16(a, bi, xlane));
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) xr[kk] = __builtin_nontemporal_load(src + 4 * kk);
}

// The same pieces as load_bf16_block, copied by the memory system straight
// into the wave's LDS slice (global_load_lds_dwordx4: lane l's 16 bytes land
// at slice[kk][l]); counted by vmcnt like any load.
__device__ __forceinline__ void prefetch_bf16_block_lds(const QuantArgs &a, const BlockIdx &bi,
                                                        int64_t xlane, u32x4 (*slice)[64]) {
  const u32x4 *src = reinterpret_cast<const u32x4 *>(x_block_bf16(a, bi, xlane));
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    __builtin_amdgcn_global_load_lds(src + 4 * kk,
                                     (__attribute__((address_space(3))) void *)&slice[kk][0], 16, 0, 0);
}

// b * 0x01010101 for b < 256: byte 0 of b in all four bytes, by a byte
// permute (a full-rate instruction; a 32-bit integer multiply issues at a
// quarter of the rate)
__device__ __forceinline__ uint32_t bytes4(uint32_t b) { return __builtin_amdgcn_perm(0u, b, 0u); }

// kRotate = false: the input is already rotated (rotation absorbed into the
// model's weights) and the MFMAs copy it through identity tiles.
// kPositions: x is a one-chunk window per (b, h); block (b, h) re-quantizes
// cache chunk pos[b] / 128 only when pos[b] % 128 == 127, i.e. when the token
// just appended at pos[b] filled its chunk (kvarn_append_rebalance).
template <bool kF32, bool kRotate, bool kPositions>
__global__ __launch_bounds__(kThreads, 4) void quantize_block_kernel(QuantArgs a) {
  __shared__ QuantSmem sm;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar LDS addresses
  const int n = lane & 15, g = lane >> 4;
  const int ti = 16 * wv + n;  // token whose input row the lane loads
  const int64_t xlane = 2 * (int64_t)ti * a.st + 16 * g;  // its bytes within a bf16 block
  const int64_t nch = a.capacity / T;
  // r' from the running maximum: the unscaled rotation's 1/sqrt(128) and the
  // 1/2 of the range step, or the 1/2 alone for pre-rotated input
  const float range_factor = kRotate ? kRangeFromUnscaled : kRangeFromRotated;

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
  u32x4 xn[4];
  uint32_t blk = blockIdx.x;
  if constexpr (!kF32) {
    if (blk < a.nblocks) {
      load_bf16_block(a, split_block(a, blk), xlane, xn);
      prefetch_bf16_block_lds(a, split_block(a, min(blk + gridDim.x, a.nblocks - 1)), xlane,
                              sm.xin[wv]);
    }
    // waited for here once, so that the loop head does not merge the first
    // loads into every block's wait
    __builtin_amdgcn_s_waitcnt(kVmcntZero);
  }
  auto rotate_f32 = [&](const BlockIdx &bi, f32x4 (&acc)[8]) {  // three bf16 terms per piece
    const u32x4 hp[4] = {sm.hop[0][lane], sm.hop[1][lane], sm.hop[2][lane], sm.hop[3][lane]};
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
    const u32x4 hp[4] = {sm.hop[0][lane], sm.hop[1][lane], sm.hop[2][lane], sm.hop[3][lane]};
    rotate_step<kRotate, 0>(acc, x[0], hp);
    rotate_step<kRotate, 1>(acc, x[1], hp);
    rotate_step<kRotate, 2>(acc, x[2], hp);
    rotate_step<kRotate, 3>(acc, x[3], hp);
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
      f32x4 acc[8];
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (kF32) {
        rotate_f32(bi, acc);
      } else {
        rotate_bf16(xn, acc);
        // first row step by Parseval: sum_j y_j^2 = 128 sum_k x_k^2 (1 sum_k
        // x_k^2 without the rotation); the diagonal of x x^T, from the same
        // operand registers, lands in lane (n, g = n / 4), register n % 4
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) gram = mfma_bf16(xn[kk], xn[kk], gram);
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
        for (int kk = 0; kk < 4; ++kk) xn[kk] = sm.xin[wv][kk][lane];
        __builtin_amdgcn_s_waitcnt((0x7 << 4) | 0xF | (0x3 << 14));  // lgkmcnt(0): reads done
        const uint32_t nb = min(blk + 2 * gridDim.x, a.nblocks - 1);
        prefetch_bf16_block_lds(a, split_block(a, nb), xlane, sm.xin[wv]);
      }
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
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
    float w[8];                  // 1/c^2 of channels 16 nt + n; 1/c after the last column step
    float cm = 1.f;  // c^2 of channel 16 wv + lane / 4 after a column step, then c
    if (a.iters > 0) {
      // v_i = 1 / (T r_i^2) of the lane's tokens. With D = T the row step's
      // 1/D and the column step's 1/T cancel: v_i = 1 / sum_j P_ij / c_j^2,
      // and the column step's weighted sum is c_j^2 itself. A zero row or
      // column (all its P are 0) takes the reciprocal of the smallest normal
      // number instead of 1: its products are 0 either way, and its stored
      // scales are set below.
      static_assert(D == T, "the row and column normalizations cancel only for square blocks");
      float v[4];
      {
        // first row step (c = 1): v_i = 1 / sum_j P_ij
        float tot;
        if constexpr (kF32) {
          float s[4];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            s[r] = ((p[r] + p[4 + r]) + (p[8 + r] + p[12 + r])) +
                   ((p[16 + r] + p[20 + r]) + (p[24 + r] + p[28 + r]));
          tot = row_reduce4<false>(s, n);
        } else {
          // token 4 g + tsel(n) sits in lane 16 g + 4 g + tsel(n), register tsel(n)
          const int r = n & 3;
          const float d = (r & 2) ? ((r & 1) ? gram.w : gram.z) : ((r & 1) ? gram.y : gram.x);
          const int t = tid;
          const int src = 20 * ((t >> 4) & 3) + tsel(t);
          tot = (kRotate ? (float)D : 1.f) * __shfl(d, src, 64);
        }
        const float vt = rcp(fmaxf(tot, kTiny));
        v[0] = token_value<0>(vt); v[1] = token_value<1>(vt);
        v[2] = token_value<2>(vt); v[3] = token_value<3>(vt);
      }
      for (int it = 0;;) {
        // column step: c_j^2 = (1/T) sum_i P_ij / r_i^2 = sum_i P_ij v_i. The
        // lane's 8 partial sums (its 4 tokens of channels 16 nt + n) go to
        // LDS; wave w then adds up channel 16 w + l / 4: lane l takes waves
        // 2 (l % 4) and 2 (l % 4) + 1, all four rows, and the quad's four
        // lanes meet by two DPP adds.
        float cp[8];
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
          cp[nt] = fmaf(p[4 * nt + 3], v[3],
                        fmaf(p[4 * nt + 2], v[2], fmaf(p[4 * nt + 1], v[1], p[4 * nt] * v[0])));
        {
          float *pw = sm.cpart + CP_WAVE * wv + lane;
#pragma unroll
          for (int nt = 0; nt < 8; ++nt) pw[CP_PLANE * nt] = cp[nt];
        }
        lds_barrier();
        {
          const float *pr = sm.cpart + CP_PLANE * wv + 2 * CP_WAVE * (lane & 3) + (lane >> 2);
          float q[8];
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) q[4 * u + r] = pr[CP_WAVE * u + 16 * r];
          cm = ((q[0] + q[1]) + (q[2] + q[3])) + ((q[4] + q[5]) + (q[6] + q[7]));
          cm += dpp_f<kXor1>(cm);
          cm += dpp_f<kXor2>(cm);
        }
        if (++it == a.iters) break;
        // 1/c^2 of channel 16 wv + l / 4 (the four lanes of each channel write
        // the same value), then every lane takes channels 16 nt + n
        sm.ctot[16 * wv + (lane >> 2)] = rcp(fmaxf(cm, kTiny));
        lds_barrier();
        {
          const float *pg = sm.ctot + n;
#pragma unroll
          for (int nt = 0; nt < 8; ++nt) w[nt] = pg[16 * nt];
        }
        // row step: r_i^2 = (1/D) sum_j P_ij / c_j^2  ->  v_i = 1 / sum_j P_ij / c_j^2
        float s[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float e = p[r] * w[0];
#pragma unroll
          for (int nt = 1; nt < 8; ++nt) e = fmaf(p[4 * nt + r], w[nt], e);
          s[r] = e;
        }
        const float tot = row_reduce4<false>(s, n);
        const float vt = rcp(fmaxf(tot, kTiny));
        v[0] = token_value<0>(vt); v[1] = token_value<1>(vt);
        v[2] = token_value<2>(vt); v[3] = token_value<3>(vt);
      }
      // c and 1/c of channel 16 wv + l / 4 (a zero column keeps c = 1)
      const float ic = cm > 0.f ? __builtin_amdgcn_rsqf(cm) : 1.f;
      cm = cm > 0.f ? cm * ic : 1.f;  // c = c^2 / sqrt(c^2)
      sm.ctot[16 * wv + (lane >> 2)] = ic;
      lds_barrier();
      {
        const float *pg = sm.ctot + (tid & 15);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) w[nt] = pg[16 * nt];
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) w[nt] = 1.f;
    }

    // ---- 4. range step and codes --------------------------------------------
    // The three global stores below (column scales, row scales, codes) are
    // issued by every wave of every block that is not skipped, each with
    // active lanes in every wave: they are the kStoresAfterPrefetch that the
    // prefetch wait counts on.
    if ((lane & 3) == 0)  // store 1 of 3; wave wv holds the column scales of channels 16 wv + [0, 16)
      a.col_scale[(bh * nch + chunk) * D + 16 * wv + ((tid & 63) >> 2)] = cm;
    float mx[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
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

    uint8_t *cbase = a.codes + (bh * nch + chunk) * CHUNK_BYTES;
    if (a.kind == KVARN_K) {
      // kw[r][k] byte i = code of token 4 g + r, channel 16 (4 k + i) + n;
      // shifted to bit 2 (n % 4) and ORed over the quad it becomes token-row
      // byte 16 k + 4 i + n / 4 (channels 4 (4 k + i) + n / 4 .. + 4)
      uint32_t kw[4][2];
      const int sh = 2 * (tid & 3);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          uint32_t c = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            c = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(y[4 * (4 * k + i) + r], qs[r], 1.5f), i, c);
          c <<= sh;
          c |= dpp_u<kXor1>(c);
          kw[r][k] = c | dpp_u<kXor2>(c);
        }
      // the four lanes of quad q hold the same words: each writes all eight
      // (token r, half k) words of the quad (equal values to equal addresses)
      const int t = tid;
      const int s = t & 3, q = (t >> 2) & 3;
      uint32_t *ks = &sm.kst[wv][0] + KST_ROW * ((t >> 4) & 3);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ks[8 * r + q] = kw[r][0];
        ks[8 * r + 4 + q] = kw[r][1];
      }
      wave_lds_sync();
      // lane n takes bytes [8 n, 8 n + 8) of the row of tokens 4 g .. 4 g + 3:
      // token n / 4 (= q), half k = s / 2, bytes 2 (s % 2) and 2 (s % 2) + 1
      // of the four quads' words
      const u32x4 wq = *reinterpret_cast<const u32x4 *>(ks + 8 * q + 4 * (s >> 1));
      const uint32_t sel = 0x05010400u + bytes4(2u * (uint32_t)(s & 1));
      const uint32_t t01 = __builtin_amdgcn_perm(wq.y, wq.x, sel);
      const uint32_t t23 = __builtin_amdgcn_perm(wq.w, wq.z, sel);
      const u32x2 pk = {__builtin_amdgcn_perm(t23, t01, 0x05040100u),
                        __builtin_amdgcn_perm(t23, t01, 0x07060302u)};
      // tokens 16 wv + 4 g + [0, 4) are 128 contiguous bytes from (16 wv + 4 g) * 32
      *reinterpret_cast<u32x2 *>(cbase + 8 * (t & 511)) = pk;  // store 3 of 3 (K)
    } else {
      // Byte j of p0 (p1) is the V byte of channel 16 j + n (16 (4 + j) + n),
      // tokens 16 wv + 4 g + [0, 4) (byte column 4 wv + g of the channel
      // row). The codes of token r of the four tiles are converted into the
      // bytes of one word, and the four tokens' words meet by shifts of 2 r
      // within the bytes (no field reaches the next byte).
      uint32_t xa[4], xb[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        xa[r] = 0;
        xb[r] = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          xa[r] = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(y[4 * j + r], qs[r], 1.5f), j, xa[r]);
          xb[r] = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(y[4 * (4 + j) + r], qs[r], 1.5f), j, xb[r]);
        }
      }
      const uint32_t p0 = (xa[0] | (xa[1] << 2)) | ((xa[2] << 4) | (xa[3] << 6));
      const uint32_t p1 = (xb[0] | (xb[1] << 2)) | ((xb[2] << 4) | (xb[3] << 6));
      // 4 x 4 byte transposes across the rows g (lanes 16 apart) of p0 and
      // p1: lane g ends with the words of tiles g and 4 + g. Rows g and g ^ 2
      // (permlane32) trade the column pair the other keeps, then rows g and
      // g ^ 1 (permlane16) the column the other keeps.
      const int t = tid;
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
      const uint32_t sel = __builtin_amdgcn_perm(
          0u, 0x06020400u, 0x03020100u ^ bytes4((uint32_t)((t >> 4) & 3)));
      // the words of channels 16 g + n (= t % 64) and 64 + 16 g + n, byte
      // column 4 wv, go through LDS so that the block leaves as 4 KB of
      // contiguous 8-byte stores
      uint32_t *vs = &sm.vst[vbuf][0];
      vs[VST_ROW * (t & 63) + (t >> 6)] = __builtin_amdgcn_perm(r2, k2, sel);
      vs[VST_ROW * ((t & 63) + 64) + (t >> 6)] = __builtin_amdgcn_perm(r2, k2, sel + 0x01010101u);
      vbuf ^= 1;
      lds_barrier();
      // thread u: channel u / 4, byte columns 8 (u % 4) + [0, 8) = the words
      // of waves 2 (u % 4) and 2 (u % 4) + 1; channel row j starts at 32 j
      const int u = tid;
      const uint32_t *src = vs + VST_ROW * (u >> 2) + 2 * (u & 3);
      const u32x2 word = {src[0], src[1]};
      *reinterpret_cast<u32x2 *>(cbase + 8 * u) = word;  // store 3 of 3 (V)
    }
  }
  // the last prefetch into the LDS slice lands before the workgroup (and its
  // LDS) goes away
  if constexpr (!kF32) __builtin_amdgcn_s_waitcnt(kVmcntZero);
}

}  // namespace

hipError_t launch_quantize(const QuantArgs &a, hipStream_t s) {
  if (a.nblocks == 0) return hipSuccess;
  // two resident workgroups per CU (register-limited); each walks blocks
  // strided by the grid
  const uint32_t resident = 2u * (uint32_t)device_cus();
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
