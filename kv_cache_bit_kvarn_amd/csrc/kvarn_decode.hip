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
// decode_split: grid (n_split, kv_heads, batch), one wave64 per workgroup,
// walking its range of 128-token chunks with an online softmax; the next
// chunk's codes and scales are loaded while the current one is computed.
// QK^T and PV run on v_mfma_f32_16x16x32_f16:
//  * code operand: a 32-bit word holds 16 codes; AND-ing it with a mask that
//    keeps one 2-bit field in each 16-bit half yields two fp16 subnormals
//    c * 4^i * 2^-24 (i = the field's position), exactly. Eight masks (one
//    shift) turn a word into the operand registers of two MFMA k-steps.
//  * the other operand (query * c_K, or p * r'_V) carries 4^-i, a power-of-
//    two range scale 2^sigma, and (query only) an fp16 hi/lo split, run as
//    two k-passes over the same code registers, so scores keep ~22 bits;
//  * the -1.5 offset of the levels is one more MFMA per chunk against a
//    constant operand that encodes code 1 in every field.
// decode_combine: grid (q_heads, batch): log-sum-exp merge of the partials
// (m, l, acc[128]), then the inverse rotation.
#include "kvarn_internal.h"

namespace kvarn {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;

// ---- code word -> fp16 subnormal operands --------------------------------
// A code word w holds codes c_0..c_15 at bits 2m. Output dwords (two fp16 each,
// low half first):
//   o[i]   = (c_i, c_{8+i}) * 4^i        i = 0..3   (k-step half 0)
//   o[4]   = (c_4, c_12)    * 4^4                   (k-step half 1)
//   o[5+i] = (c_{5+i}, c_{13+i}) * 4^i  i = 0..2   (k-step half 1)
// all times 2^-24. The field scale of code index c is 4^f(c % 8) with
// f = {0, 1, 2, 3, 4, 0, 1, 2}.
__device__ __forceinline__ void unpack_codes(uint32_t w, u32x4 &h0, u32x4 &h1) {
  const uint32_t x = w >> 10;
  h0[0] = w & 0x00030003u;
  h0[1] = w & 0x000C000Cu;
  h0[2] = w & 0x00300030u;
  h0[3] = w & 0x00C000C0u;
  h1[0] = w & 0x03000300u;
  h1[1] = x & 0x00030003u;
  h1[2] = x & 0x000C000Cu;
  h1[3] = x & 0x00300030u;
}

__host__ __device__ constexpr int field_exp(int c) {  // f(c % 8)
  return (c & 7) < 5 ? (c & 7) : (c & 7) - 5;
}

// code index (0..15 within a word) held by k-slot e of k-step half hs
__device__ __forceinline__ int slot_code(int hs, int e) {
  if (hs == 0) return (e & 1) ? 8 + (e >> 1) : (e >> 1);
  if (e < 2) return e ? 12 : 4;
  return (e & 1) ? 13 + ((e - 3) >> 1) : 5 + ((e - 2) >> 1);
}

// lane-group g (0..3) covers code words 2g, 2g+1 of a row, i.e. elements
// [32 g, 32 g + 32); k-step s (0..3) takes word 2g + (s >> 1), half s & 1.
__device__ __forceinline__ int kslot_elem(int g, int s, int e) {
  return 32 * g + 16 * (s >> 1) + slot_code(s & 1, e);
}

// position of element j in the [g][s][e] order of kslot_elem
__device__ __forceinline__ int elem_slot_pos(int j) {
  const int g = j >> 5, w = (j >> 4) & 1, c = j & 15;
  int hs, e;
  if (c < 4) { hs = 0; e = 2 * c; }
  else if (c >= 8 && c < 12) { hs = 0; e = 2 * (c - 8) + 1; }
  else if (c == 4) { hs = 1; e = 0; }
  else if (c == 12) { hs = 1; e = 1; }
  else if (c < 8) { hs = 1; e = 2 + 2 * (c - 5); }
  else { hs = 1; e = 3 + 2 * (c - 13); }
  return ((g * 4) + 2 * w + hs) * 8 + e;
}

__device__ __forceinline__ f16x8 as_f16x8(u32x4 v) { return __builtin_bit_cast(f16x8, v); }

__device__ __forceinline__ uint32_t pack_rtz(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

__device__ __forceinline__ f32x4 mfma(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

// power-of-two scale 2^sigma with max * 2^sigma in [2^14, 2^15) (1 if max == 0)
__device__ __forceinline__ float range_scale(float mx, int &sigma) {
  sigma = 0;
  if (mx > 0.f) {
    sigma = 15 - __builtin_amdgcn_frexp_expf(mx);
    sigma = sigma > 100 ? 100 : (sigma < -100 ? -100 : sigma);
  }
  return __builtin_ldexpf(1.f, sigma);
}

// In-place Sylvester Hadamard transform (unscaled) of rows x[n][128] in LDS.
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

// ---- cross-lane reductions on DPP (no LDS round trip) ----------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int kQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// max / sum over aligned groups of N lanes (N = 8 or 16); every lane gets it
template <int N>
__device__ __forceinline__ float group_max(float v) {
  v = fmaxf(v, dpp<kQuadSwap1>(v));
  v = fmaxf(v, dpp<kQuadSwap2>(v));
  v = fmaxf(v, dpp<kRowHalfMirror>(v));
  if constexpr (N == 16) v = fmaxf(v, dpp<kRowMirror>(v));
  return v;
}
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp<kQuadSwap1>(v);
  v += dpp<kQuadSwap2>(v);
  v += dpp<kRowHalfMirror>(v);
  if constexpr (N == 16) v += dpp<kRowMirror>(v);
  return v;
}
// max over the wave, wave-uniform result
__device__ __forceinline__ float wave_max_u(float v) {
  v = group_max<16>(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Per-head rows are padded by 4 words so that rows of different heads start
// on different LDS banks.
constexpr int SC_PITCH = T + 4;       // floats per head row of sc
constexpr int OP_PITCH = 4 * 4 * 4 + 4;  // words per head row of an operand array

// LDS position of token t in the per-token arrays (sc, rk, rv): inside each
// 16-token tile the four 4-token quads are permuted by an XOR that depends on
// the tile pair, so that the softmax lanes' 16-byte reads (one tile per lane,
// 8 lanes per LDS cycle) fall on distinct banks. Quads stay contiguous.
__host__ __device__ constexpr int quad_swz(int tile) {  // {0, 2, 1, 3}[(tile >> 1) & 3]
  return (((tile >> 1) & 1) << 1) | ((tile >> 2) & 1);
}
__host__ __device__ constexpr int tok_pos(int t) {
  return (t & ~15) | ((((t >> 2) & 3) ^ quad_swz(t >> 4)) << 2) | (t & 3);
}
// Word offset of operand quad Q = 4 g + s (lane group g, k-step s) in a head
// row of ahi/alo/ap: quads Q and Q + 8 are moved to different banks for the
// softmax lanes' P' writes.
__host__ __device__ constexpr int op_quad(int q) { return 4 * (q ^ ((q >> 3) & 1)); }

template <int GP>
struct alignas(16) DecSmem {
  alignas(16) float qt[GP][D];            // rotated, scaled query (setup only)
  alignas(16) float ck[D];                // c_K in [g][s][e] order
  alignas(16) float cv[16][9];            // cv[n][ct] = c_V[16 ct + n] (odd pitch)
  alignas(16) float rk[T];                // r'_K, tok_pos order
  alignas(16) float rv[T];                // r'_V * 4^-f(t % 8), tok_pos order
  alignas(16) float sc[GP][SC_PITCH];     // QK results (offset already removed), tok_pos order
  alignas(16) uint32_t ahi[GP][OP_PITCH]; // query operand, fp16 pairs, [m][(g * 4 + s) * 4 + dword]
  alignas(16) uint32_t alo[GP][OP_PITCH];
  alignas(16) uint32_t ap[GP][OP_PITCH];  // P' operand, same layout
  float alpha[GP];
};

struct ChunkRegs {
  u32x2 k[8];  // K code words 2g, 2g+1 of token 16 tau + n
  u32x2 v[8];  // V code words 2g, 2g+1 of channel 16 ct + n
  u32x2 ck, cv, rk, rv;  // scales of elements 2l, 2l+1
};

__device__ __forceinline__ void load_chunk(const DecodeArgs &a, int64_t bg, int64_t nchunks, int k,
                                           int lane, ChunkRegs &r) {
  const int64_t chunk = bg * nchunks + k;
  const int n = lane & 15, g = lane >> 4;
  const uint8_t *kc = a.k_codes + chunk * CHUNK_BYTES + n * 32 + 8 * g;
  const uint8_t *vc = a.v_codes + chunk * CHUNK_BYTES + n * 32 + 8 * g;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    r.k[t] = *reinterpret_cast<const u32x2 *>(kc + t * 16 * 32);
    r.v[t] = *reinterpret_cast<const u32x2 *>(vc + t * 16 * 32);
  }
  r.ck = *reinterpret_cast<const u32x2 *>(a.k_col + chunk * D + 2 * lane);
  r.cv = *reinterpret_cast<const u32x2 *>(a.v_col + chunk * D + 2 * lane);
  const int64_t row = bg * (int64_t)a.capacity + (int64_t)k * T + 2 * lane;
  r.rk = *reinterpret_cast<const u32x2 *>(a.k_row + row);
  r.rv = *reinterpret_cast<const u32x2 *>(a.v_row + row);
}

// Per-lane state of one decode_split workgroup (one wave).
template <int GP>
struct SplitState {
  static constexpr int NU = GP / 4;      // query-operand units per lane
  static constexpr int LPH = 64 / GP;    // softmax lanes per head
  static constexpr int NHW = 16 / LPH;   // half code words (8 tokens) per softmax lane
  float qh[NU][8];                       // query * scales for this lane's units
  f32x4 acc[8];                          // PV accumulators (rows = heads 4 lg + r)
  float m_run, l_run;
};

template <int GP>
__device__ __forceinline__ void process_chunk(const DecodeArgs &a, DecSmem<GP> &sm,
                                              SplitState<GP> &st, const ChunkRegs &cur, int k,
                                              int len, int lane, const u32x4 &one0,
                                              const u32x4 &one1) {
  constexpr int NU = SplitState<GP>::NU, LPH = SplitState<GP>::LPH, NHW = SplitState<GP>::NHW;
  const int n = lane & 15, lg = lane >> 4;
  const int gu = (lane >> 2) & 3, su = lane >> 4;
  const int sh = lane / LPH;             // softmax head of this lane
  const int nvalid = min(len - k * T, T);

  // ---- scales to LDS ----
  __syncthreads();  // previous chunk's LDS readers are done
  sm.ck[elem_slot_pos(2 * lane)] = __uint_as_float(cur.ck[0]);
  sm.ck[elem_slot_pos(2 * lane + 1)] = __uint_as_float(cur.ck[1]);
  sm.cv[(2 * lane) & 15][(2 * lane) >> 4] = __uint_as_float(cur.cv[0]);
  sm.cv[(2 * lane + 1) & 15][(2 * lane + 1) >> 4] = __uint_as_float(cur.cv[1]);
  const int tp = tok_pos(2 * lane);  // 2 lane and 2 lane + 1 stay adjacent
  sm.rk[tp] = __uint_as_float(cur.rk[0]);
  sm.rk[tp + 1] = __uint_as_float(cur.rk[1]);
  const float rv0 = 2 * lane < nvalid ? __uint_as_float(cur.rv[0]) : 0.f;
  const float rv1 = 2 * lane + 1 < nvalid ? __uint_as_float(cur.rv[1]) : 0.f;
  int sig_v;
  const float sv = range_scale(wave_max_u(fmaxf(rv0, rv1)), sig_v);
  sm.rv[tp] = rv0 * sv * __builtin_ldexpf(1.f, -2 * field_exp(2 * lane));
  sm.rv[tp + 1] = rv1 * sv * __builtin_ldexpf(1.f, -2 * field_exp(2 * lane + 1));
  __syncthreads();

  // ---- query operand: a = q * c_K * 2^sigma_q, fp16 hi/lo ----
  int sig_q;
  {
    const f32x4 c0v = *reinterpret_cast<const f32x4 *>(&sm.ck[(gu * 4 + su) * 8]);
    const f32x4 c1v = *reinterpret_cast<const f32x4 *>(&sm.ck[(gu * 4 + su) * 8 + 4]);
    const float cc[8] = {c0v.x, c0v.y, c0v.z, c0v.w, c1v.x, c1v.y, c1v.z, c1v.w};
    float av[NU][8];
    float mx = 0.f;
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        av[u][e] = st.qh[u][e] * cc[e];
        mx = fmaxf(mx, fabsf(av[u][e]));
      }
    const float sq = range_scale(wave_max_u(mx), sig_q);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      u32x4 hi, lo;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        // hi = x truncated to fp16's 11 significant bits (exact in fp32 and,
        // for |x| in the fp16 normal range, exact in fp16); lo = x - hi.
        // Formed in fp32 so that no f16 -> f32 read-back of the packed hi
        // pair exists (that pattern was mis-fused into v_fma_mix_f32 with
        // the wrong source register by this compiler).
        const float x0 = av[u][2 * d] * sq, x1 = av[u][2 * d + 1] * sq;
        const float h0 = __uint_as_float(__float_as_uint(x0) & 0xFFFFE000u);
        const float h1 = __uint_as_float(__float_as_uint(x1) & 0xFFFFE000u);
        hi[d] = pack_rtz(h0, h1);
        lo[d] = pack_rtz(x0 - h0, x1 - h1);
      }
      const int mu = (lane & 3) + 4 * u;
      *reinterpret_cast<u32x4 *>(&sm.ahi[mu][op_quad(gu * 4 + su)]) = hi;
      *reinterpret_cast<u32x4 *>(&sm.alo[mu][op_quad(gu * 4 + su)]) = lo;
    }
  }
  __syncthreads();
  u32x4 ahi[4], alo[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    ahi[s] = n < GP ? *reinterpret_cast<const u32x4 *>(&sm.ahi[n][op_quad(lg * 4 + s)]) : u32x4{0u, 0u, 0u, 0u};
    alo[s] = n < GP ? *reinterpret_cast<const u32x4 *>(&sm.alo[n][op_quad(lg * 4 + s)]) : u32x4{0u, 0u, 0u, 0u};
  }

  // ---- QK^T: offset term first, then 8 token tiles x (4 hi + 4 lo) k-steps
  // started from -1.5 * offset, so D = sum_j a_j (code_tj - 1.5) directly ----
  {
    f32x4 off = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      off = mfma(as_f16x8(ahi[s]), as_f16x8((s & 1) ? one1 : one0), off);
      off = mfma(as_f16x8(alo[s]), as_f16x8((s & 1) ? one1 : one0), off);
    }
    off *= -1.5f;
#pragma unroll
    for (int tau = 0; tau < 8; ++tau) {
      u32x4 b0, b1, b2, b3;
      unpack_codes(cur.k[tau][0], b0, b1);
      unpack_codes(cur.k[tau][1], b2, b3);
      f32x4 d = mfma(as_f16x8(ahi[0]), as_f16x8(b0), off);
      d = mfma(as_f16x8(ahi[1]), as_f16x8(b1), d);
      d = mfma(as_f16x8(ahi[2]), as_f16x8(b2), d);
      d = mfma(as_f16x8(ahi[3]), as_f16x8(b3), d);
      d = mfma(as_f16x8(alo[0]), as_f16x8(b0), d);
      d = mfma(as_f16x8(alo[1]), as_f16x8(b1), d);
      d = mfma(as_f16x8(alo[2]), as_f16x8(b2), d);
      d = mfma(as_f16x8(alo[3]), as_f16x8(b3), d);
      if (lg < GP / 4) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sm.sc[4 * lg + r][16 * tau + (n ^ (quad_swz(tau) << 2))] = d[r];
      }
    }
  }
  __syncthreads();

  // ---- online softmax. A lane owns NHW half code words of head sh: the
  // tokens 16 w + 4 hs + i and 16 w + 8 + 4 hs + i (i < 4), i.e. exactly
  // the fp16 pairs of one P' operand dword quad ----
  {
    const float kscale = __builtin_ldexpf(1.f, 24 - sig_q);
    float s[NHW][8];
    float mc = -INFINITY;
#pragma unroll
    for (int j = 0; j < NHW; ++j) {
      const int hw = (lane % LPH) * NHW + j;      // half-word index 0..15
      const int t1 = 16 * (hw >> 1) + 4 * (hw & 1);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int t = t1 + 8 * q;
        const f32x4 raw = *reinterpret_cast<const f32x4 *>(&sm.sc[sh][tok_pos(t)]);
        const f32x4 rk4 = *reinterpret_cast<const f32x4 *>(&sm.rk[tok_pos(t)]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = raw[i] * (rk4[i] * kscale);
          s[j][4 * q + i] = t + i < nvalid ? v : -INFINITY;
          mc = fmaxf(mc, s[j][4 * q + i]);
        }
      }
    }
    mc = group_max<LPH>(mc);
    // integer running max (log2 units): P' of a chunk then differs between
    // split layouts only by powers of two, so its fp16 rounding does not
    const float mn = fmaxf(st.m_run, ceilf(mc));
    const float al = mn == -INFINITY ? 1.f : exp2f(st.m_run - mn);
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < NHW; ++j) {
      const int hw = (lane % LPH) * NHW + j;
      const int t1 = 16 * (hw >> 1) + 4 * (hw & 1);
      const f32x4 rva = *reinterpret_cast<const f32x4 *>(&sm.rv[tok_pos(t1)]);
      const f32x4 rvb = *reinterpret_cast<const f32x4 *>(&sm.rv[tok_pos(t1 + 8)]);
      u32x4 pk;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pa = mn == -INFINITY ? 0.f : exp2f(s[j][i] - mn);
        const float pb = mn == -INFINITY ? 0.f : exp2f(s[j][4 + i] - mn);
        ps += pa + pb;
        pk[i] = pack_rtz(pa * rva[i], pb * rvb[i]);
      }
      // dword quad (word hw >> 1, half hw & 1) of the P' operand of head sh:
      // lane group g = word >> 1, k-step s = 2 (word & 1) + half
      const int w = hw >> 1;
      *reinterpret_cast<u32x4 *>(&sm.ap[sh][op_quad((w >> 1) * 4 + 2 * (w & 1) + (hw & 1))]) = pk;
    }
    st.l_run = st.l_run * al + ps;
    st.m_run = mn;
    if (lane % LPH == 0) sm.alpha[sh] = al;
  }
  __syncthreads();

  // ---- PV: 8 channel tiles x 4 k-steps, started from -1.5 * offset ----
  {
    u32x4 ap[4];
#pragma unroll
    for (int s = 0; s < 4; ++s)
      ap[s] = n < GP ? *reinterpret_cast<const u32x4 *>(&sm.ap[n][op_quad(lg * 4 + s)]) : u32x4{0u, 0u, 0u, 0u};
    f32x4 off = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) off = mfma(as_f16x8(ap[s]), as_f16x8((s & 1) ? one1 : one0), off);
    off *= -1.5f;
    f32x4 alr;
#pragma unroll
    for (int r = 0; r < 4; ++r) alr[r] = (4 * lg + r < GP) ? sm.alpha[4 * lg + r] : 1.f;
    // the running max moves by whole powers of two: rescale only when it moved
    if (alr[0] != 1.f || alr[1] != 1.f || alr[2] != 1.f || alr[3] != 1.f) {
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) st.acc[ct] *= alr;
    }
    const float vscale = __builtin_ldexpf(1.f, 24 - sig_v);
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
      u32x4 b0, b1, b2, b3;
      unpack_codes(cur.v[ct][0], b0, b1);
      unpack_codes(cur.v[ct][1], b2, b3);
      f32x4 d = mfma(as_f16x8(ap[0]), as_f16x8(b0), off);
      d = mfma(as_f16x8(ap[1]), as_f16x8(b1), d);
      d = mfma(as_f16x8(ap[2]), as_f16x8(b2), d);
      d = mfma(as_f16x8(ap[3]), as_f16x8(b3), d);
      const float cvs = sm.cv[n][ct] * vscale;
#pragma unroll
      for (int r = 0; r < 4; ++r) st.acc[ct][r] = fmaf(cvs, d[r], st.acc[ct][r]);
    }
  }
}

template <int GP>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs a) {
  __shared__ DecSmem<GP> sm;
  constexpr int NU = SplitState<GP>::NU, LPH = SplitState<GP>::LPH;
  const int lane = threadIdx.x;
  const int split = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = a.q_heads / a.kv_heads;
  const int nch = a.capacity / T;
  const int len = a.lens[b];
  const bool valid = len >= 1 && len <= a.capacity;
  const int used = valid ? (len + T - 1) / T : 0;
  const int per = (nch + a.n_split - 1) / a.n_split;
  const int c0 = split * per;
  const int c1 = min(c0 + per, used);
  const int64_t bg = (int64_t)b * a.kv_heads + g;

  // ---- query: rotate; fold softmax scale, log2(e), 1/sqrt(128), 4^-f -----
  for (int idx = lane; idx < GP * D; idx += 64) {
    const int m = idx / D, j = idx - m * D;
    sm.qt[m][j] = m < G ? load_q(a.q, a.q_dtype, ((int64_t)b * a.q_heads + g * G + m) * D + j) : 0.f;
  }
  __syncthreads();
  lds_fwht_rows(&sm.qt[0][0], GP);
  SplitState<GP> st;
  {
    const int gu = (lane >> 2) & 3, su = lane >> 4;
    const float qs = a.scale * kLog2e * kInvSqrtD;
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = kslot_elem(gu, su, e);
        st.qh[u][e] = sm.qt[(lane & 3) + 4 * u][j] * qs * __builtin_ldexpf(1.f, -2 * field_exp(j));
      }
  }
#pragma unroll
  for (int ct = 0; ct < 8; ++ct) st.acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m_run = -INFINITY;
  st.l_run = 0.f;
  // constant operand: code 1 in every field (the level offset term)
  u32x4 one0, one1;
  unpack_codes(0x55555555u, one0, one1);

  // chunks [c0, c1); the next chunk's loads are in flight while the current
  // one is computed
  ChunkRegs cur, nxt;
  if (c0 < c1) load_chunk(a, bg, nch, c0, lane, cur);
  for (int k = c0; k < c1; ++k) {
    if (k + 1 < c1) load_chunk(a, bg, nch, k + 1, lane, nxt);
    process_chunk<GP>(a, sm, st, cur, k, len, lane, one0, one1);
    cur = nxt;
  }

  // ---- partial results: (m, l, acc) per query head of this split ----
  const int sh = lane / LPH;
  const float lsum = group_sum<LPH>(st.l_run);
  const int n = lane & 15, lg = lane >> 4;
  if (lane % LPH == 0 && sh < G) {
    float *pp = a.partial + (((int64_t)b * a.q_heads + g * G + sh) * a.n_split + split) * (2 + D);
    pp[0] = st.m_run;
    pp[1] = lsum;
  }
  if (lg < GP / 4) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 4 * lg + r;
      if (h < G) {
        float *pp = a.partial + (((int64_t)b * a.q_heads + g * G + h) * a.n_split + split) * (2 + D);
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) pp[2 + 16 * ct + n] = st.acc[ct][r];
      }
    }
  }
}

// Log-sum-exp merge of the split partials of one (sequence, query head), then
// the inverse rotation. Thread s < n_split first reads split s's (m, l); the
// block reduces the maximum and the weighted denominator; then every thread
// (one output channel) walks the splits with independent, coalesced loads.
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a) {
  __shared__ float o[D];
  __shared__ float wgt[D];
  __shared__ float red[4];
  const int h = blockIdx.x, b = blockIdx.y, j = threadIdx.x;
  const float *pp = a.partial + ((int64_t)b * a.q_heads + h) * a.n_split * (2 + D);
  // pass 1: maximum of the split maxima
  float mx = -INFINITY;
  for (int s = j; s < a.n_split; s += D) mx = fmaxf(mx, pp[(int64_t)s * (2 + D)]);
  mx = group_max<16>(mx);
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  if ((j & 63) == 0) red[j >> 6] = mx;
  __syncthreads();
  const float M = fmaxf(red[0], red[1]);
  // pass 2: weights, denominator and numerator
  float num = 0.f, den = 0.f;
  if (M != -INFINITY) {
    for (int base = 0; base < a.n_split; base += D) {
      const int s = base + j;
      float w = 0.f;
      if (s < a.n_split) {
        const float ms = pp[(int64_t)s * (2 + D)];
        w = ms == -INFINITY ? 0.f : exp2f(ms - M);
        den += w * pp[(int64_t)s * (2 + D) + 1];
      }
      __syncthreads();  // previous round's readers of wgt are done
      wgt[j] = w;
      __syncthreads();
      const int cnt = min(D, a.n_split - base);
      const float *col = pp + (int64_t)base * (2 + D) + 2 + j;
#pragma unroll 8
      for (int q = 0; q < cnt; ++q) num += wgt[q] * col[(int64_t)q * (2 + D)];
    }
  }
  den = group_sum<16>(den);
  den += __shfl_xor(den, 16, 64);
  den += __shfl_xor(den, 32, 64);
  __syncthreads();
  if ((j & 63) == 0) red[2 + (j >> 6)] = den;
  __syncthreads();
  den = red[2] + red[3];
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
  // about 4096 single-wave workgroups: 16 per CU on 256 CUs
  int s = (4096 + pairs - 1) / pairs;
  if (s > nch) s = nch;
  if (s < 1) s = 1;
  return s;
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
  if (a.batch == 0 || a.q_heads == 0) return hipSuccess;
  const dim3 grid(a.n_split, a.kv_heads, a.batch);
  if (a.q_heads / a.kv_heads <= 4)
    hipLaunchKernelGGL(decode_split_kernel<4>, grid, dim3(64), 0, s, a);
  else
    hipLaunchKernelGGL(decode_split_kernel<8>, grid, dim3(64), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(a.q_heads, a.batch), dim3(D), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvarn
