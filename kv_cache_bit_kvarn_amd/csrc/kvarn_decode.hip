// Decode attention over the 2-bit KVarN cache on gfx950, both scales fused
// into the dequantization (rndamp article on KVarN, "Numbers").
//
// Rotated-domain evaluation. With H = H_D / sqrt(D) (symmetric, orthogonal)
// the cache stores y_hat = x_hat H, so
//   <q, x_hat_t>      = <q H, y_hat_t>
//                     = r'_t * sum_j (qH)_j c_j (code_tj - 1.5)
//   sum_t p_t x_hat_t = ( sum_t p_t y_hat_t ) H
//                     = ( c_j * sum_t (p_t r'_t)(code_tj - 1.5) )_j  H.
// The query is rotated once per wave, the column scale of K is folded into
// the rotated query per chunk, the row scale of K into each score, the row
// scale of V into each probability, and the column scale of V into the
// output; the output is rotated back after the split-KV merge.
//
// One launch, grid (n_wg * head_groups, kv_heads, batch): a workgroup is four
// waves, each a split serving up to 4 query heads of one kv-head over its
// range of 128-token chunks with an online softmax; the next chunk's codes
// and scales are loaded while the current one is computed. The waves merge
// in LDS, and the last workgroup of a row merges the row's partials (no
// second launch). Both products run on v_mfma_scale_f32_16x16x128_f8f6f4,
// the cache codes being its fp4 operand:
//  * a 2-bit code c in the low bits of a 4-bit field is the e2m1 number c/2,
//    so w & 0x33333333 and (w >> 2) & 0x33333333 turn a code word into two
//    operand registers (16 codes for 3 instructions), and c/2 - 3/4 is half
//    the level c - 1.5;
//  * the other operand (query * c_K, or p * r'_V) is fp8 e4m3, written as a
//    sum of terms x = t0 + t1 + ... where each term is the fp8 rounding of
//    what the earlier ones left (4 terms, ~16 significant bits, for the query;
//    3 terms, ~12 bits, for the probabilities). Row 4 h + k of the 16-row
//    operand holds term k of head h, so one MFMA covers 16 tokens (QK) or 16
//    channels (PV) for all heads and terms, and the terms of a head land in
//    the four accumulator registers of one lane;
//  * a per-head power-of-two range scale (largest magnitude in [128, 256))
//    is undone by the MFMA's per-row E8M0 scale;
//  * the level offset is one MFMA per chunk against a constant -1.5 operand
//    at scale 2^-1, added to each head's term sum.
// Head sizes 64, 128 and 256 share the kernel: the QK contraction runs over
// 128-channel halves (a 64-channel head fills half of one, the rest of both
// operands zero) and PV over D / 16 channel tiles.
#include <atomic>
#include <mutex>

#include "kvarn_internal.h"

namespace kvarn {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int HG = 4;                       // query heads per wave (and per workgroup)
constexpr int kDecWaves = KVARN_DECODE_WAVES;  // waves (splits) per workgroup
constexpr uint32_t kFieldMask = 0x33333333u;  // low 2 bits of every 4-bit field
constexpr uint32_t kFp4Neg3Half = 0xBBBBBBBBu;  // e2m1 -1.5 in every field

// ---- the k order shared by both MFMA operands -----------------------------
// fp8 operand (8 dwords per lane, lane = row + 16 g): byte e holds
//   k = 16 g + e (e < 16),  k = 48 + 16 g + e (e >= 16).
// fp4 operand (4 dwords per lane, lane = column + 16 g): field e holds
//   k = 32 g + e.
// A code row (a token of K, a channel of V: 32 bytes) gives lane group g its
// bytes [8 g, 8 g + 8) = words w0, w1, unpacked to the dwords
//   w0 & M, (w0 >> 2) & M, w1 & M, (w1 >> 2) & M,
// so field i of dword d carries code 32 g + 16 (d >> 1) + 2 i + (d & 1) of
// the row. k_elem(k) is therefore the channel (QK) or token (PV) at index k.
__host__ __device__ constexpr int k_elem(int k) {
  return 32 * (k >> 5) + 16 * ((k >> 4) & 1) + 2 * (k & 7) + ((k >> 3) & 1);
}
__host__ __device__ constexpr int fp8_k(int g, int e) { return e < 16 ? 16 * g + e : 48 + 16 * g + e; }

// The fp8 operand is built in 8-byte packets: slot s = 4 g + p is bytes
// [8 p, 8 p + 8) of lane group g, and its byte j holds element
// slot_elem(s, j) = 16 (s >> 2) + 64 ((s >> 1) & 1) + (s & 1) + 2 j.
// Slot s is also the output column of the lane that computes it, so the
// softmax lane of column s finds exactly the scores of its P' packet.
__host__ __device__ constexpr int slot_elem(int s, int j) {
  return k_elem(fp8_k(s >> 2, 8 * (s & 3) + j));
}
__host__ __device__ constexpr int elem_slot(int x) { return 4 * ((x >> 4) & 3) + 2 * (x >> 6) + (x & 1); }
__host__ __device__ constexpr int elem_j(int x) { return (x >> 1) & 7; }
// Per-element LDS arrays read slot-wise: 8 floats per slot and 4 floats of
// padding after every 4 slots, so 16-byte reads by 8 lanes hit distinct banks.
__host__ __device__ constexpr int slot_base(int s) { return 8 * s + 4 * (s >> 2); }
__host__ __device__ constexpr int elem_pos(int x) { return slot_base(elem_slot(x)) + elem_j(x); }
constexpr int SLOT_ARRAY = 8 * 16 + 4 * 4;
constexpr int OP_ROW = 36;  // dwords per operand row: 4 lane groups x 8 + 4 padding

__host__ __device__ constexpr bool check_maps() {
  bool seen[D] = {};
  for (int k = 0; k < D; ++k) {
    const int e = k_elem(k);
    if (e < 0 || e >= D || seen[e]) return false;
    seen[e] = true;
  }
  for (int g = 0; g < 4; ++g)
    for (int e = 0; e < 32; ++e) {
      const int s = 4 * g + (e >> 3), j = e & 7, x = slot_elem(s, j);
      if (x != 16 * (s >> 2) + 64 * ((s >> 1) & 1) + (s & 1) + 2 * j) return false;
      if (elem_slot(x) != s || elem_j(x) != j) return false;
    }
  return true;
}
static_assert(check_maps(), "operand index maps are not consistent");

// D = (A * 2^(scale_a - 127)) (B * 2^(SCALE_B - 127)) + C
template <int SCALE_B = 127>
__device__ __forceinline__ f32x4 mfma_f8f4(const u32x8 &a, const u32x4 &b, const f32x4 &c,
                                           int scale_a) {
  const i32x8 av = __builtin_bit_cast(i32x8, a);
  const i32x8 bv = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  // A: fp8 e4m3 (format 0), B: fp4 e2m1 (format 4)
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 4, 0, scale_a, 0, SCALE_B);
}

// -3/4 * (row sums of A): the level offset, as the accumulator input
__device__ __forceinline__ f32x4 level_offset(const u32x8 &a, int scale_a) {
  const u32x4 neg = {kFp4Neg3Half, kFp4Neg3Half, kFp4Neg3Half, kFp4Neg3Half};
  return mfma_f8f4<126>(a, neg, f32x4{0.f, 0.f, 0.f, 0.f}, scale_a);  // -1.5 * 2^-1
}

__device__ __forceinline__ u32x4 code_operand(const u32x2 &w) {
  return u32x4{w[0] & kFieldMask, (w[0] >> 2) & kFieldMask, w[1] & kFieldMask,
               (w[1] >> 2) & kFieldMask};
}

// x (|x| < 448) as NT fp8 terms; term k of the 8 values, in order, in out[k].
template <int NT>
__device__ __forceinline__ void fp8_terms(float (&x)[8], u32x2 (&out)[NT]) {
#pragma unroll
  for (int k = 0; k < NT; ++k) {
    uint32_t w0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], 0u, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], w0, true);
    uint32_t w1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[4], x[5], 0u, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(x[6], x[7], w1, true);
    out[k] = u32x2{w0, w1};
    if (k + 1 < NT) {
      const f32x2 b0 = __builtin_amdgcn_cvt_pk_f32_fp8(w0, false);
      const f32x2 b1 = __builtin_amdgcn_cvt_pk_f32_fp8(w0, true);
      const f32x2 b2 = __builtin_amdgcn_cvt_pk_f32_fp8(w1, false);
      const f32x2 b3 = __builtin_amdgcn_cvt_pk_f32_fp8(w1, true);
      x[0] -= b0[0];
      x[1] -= b0[1];
      x[2] -= b1[0];
      x[3] -= b1[1];
      x[4] -= b2[0];
      x[5] -= b2[1];
      x[6] -= b3[0];
      x[7] -= b3[1];
    }
  }
}

// exponent sigma with mx * 2^sigma in [128, 256) (0 when mx is 0)
__device__ __forceinline__ int range_exp8(float mx) {
  if (!(mx > 0.f)) return 0;
  const int s = 8 - __builtin_amdgcn_frexp_expf(mx);
  return s > 100 ? 100 : (s < -100 ? -100 : s);
}

// E8M0 scale byte 2^-sigma_h for the operand rows of this lane (head
// (lane >> 2) & 3); sigma is uniform over each 16-lane row h.
__device__ __forceinline__ int row_scale_byte(int sigma, int lane) {
  const int s0 = __builtin_amdgcn_readlane(sigma, 0);
  const int s1 = __builtin_amdgcn_readlane(sigma, 16);
  const int s2 = __builtin_amdgcn_readlane(sigma, 32);
  const int s3 = __builtin_amdgcn_readlane(sigma, 48);
  const int h = (lane >> 2) & 3;
  const int s = h == 0 ? s0 : (h == 1 ? s1 : (h == 2 ? s2 : s3));
  return 127 - s;
}

// Each wave exchanges values between its lanes through LDS of its own, and
// the LDS accesses of one wave are performed in program order: such an
// exchange needs only a wavefront-scope fence (which keeps the compiler from
// reordering the accesses), not a barrier or a wait for the writes to
// complete.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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

// Sizes of the kernel for head size DD (64, 128 or 256). The QK contraction
// runs over 128-channel halves (one MFMA each: DD = 256 has two; DD = 64 uses
// the first 64 channels of one, the rest of its operands zero); PV writes
// 16-channel output tiles.
template <int DD>
struct Dims {
  static_assert(DD == 64 || DD == 128 || DD == 256, "head size");
  static constexpr int NQ = DD > 128 ? 2 : 1;  // QK halves
  static constexpr int NCT = DD / 16;          // PV output tiles
  static constexpr int KROW = DD / 4;          // bytes of a K token row
  static constexpr int CB = T * DD / 4;        // code bytes of a chunk
  static constexpr int CPL = DD / 64;          // column scales (and output channels) per lane
  static constexpr int CV_ARRAY = NCT * 16 + 16;
};
// c_V in LDS: channel c is read by the lanes of output column c % 16, tile
// c / 16; NCT floats per column and 4 floats of padding after every 4
// columns (for NCT = 8 this is slot_base, as for the other scale arrays)
__host__ __device__ constexpr int cv_base(int nct, int s) { return nct * s + 4 * (s >> 2); }
static_assert(cv_base(8, 5) == slot_base(5) && cv_base(8, 12) == slot_base(12), "c_V layout");

template <int DD>
struct DecSmem {
  alignas(16) float ck[Dims<DD>::NQ][SLOT_ARRAY];  // c_K per half, elem_pos order
  alignas(16) float cv[Dims<DD>::CV_ARRAY];        // c_V, cv_base order
  alignas(16) float rk[SLOT_ARRAY];                // r'_K, elem_pos order
  alignas(16) float rv[SLOT_ARRAY];                // r'_V, elem_pos order
  alignas(16) uint32_t aq[Dims<DD>::NQ][16][OP_ROW];  // QK fp8 operand per half, row 4 h + k
  alignas(16) uint32_t ap[16][OP_ROW];             // PV fp8 operand, rows 4 h + 3 stay zero
};

// Codes and scales of one chunk, in the lane's operand order.
template <int DD>
struct ChunkRegs {
  u32x2 k[Dims<DD>::NQ][8];  // K bytes [8 g, 8 g + 8) of half hf of token slot_elem(n, tau)
  u32x2 v[Dims<DD>::NCT];    // V bytes [8 g, 8 g + 8) of channel 16 ct + n
  float ck[Dims<DD>::CPL], cv[Dims<DD>::CPL];  // column scales of channels CPL lane + i
  u32x2 rk, rv;              // row scales of tokens 2 lane, 2 lane + 1
};

// The cache is streamed once per decode step: non-temporal loads, which keep
// it from displacing reused lines in the caches.
template <typename V>
__device__ __forceinline__ V stream_load(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const V *>(p));
}

template <int N>
__device__ __forceinline__ void load_floats(const float *p, float (&out)[N]) {
  if constexpr (N == 1) {
    out[0] = stream_load<float>(p);
  } else if constexpr (N == 2) {
    const u32x2 u = stream_load<u32x2>(p);
    out[0] = __uint_as_float(u[0]);
    out[1] = __uint_as_float(u[1]);
  } else {
    static_assert(N == 4, "column scales per lane");
    const u32x4 u = stream_load<u32x4>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(u[i]);
  }
}

template <int DD, bool kTwoScales>
__device__ __forceinline__ void load_chunk(const DecodeArgs &a, int64_t bg, int64_t nchunks,
                                           int k, int lane, ChunkRegs<DD> &r) {
  using Dm = Dims<DD>;
  const int64_t chunk = bg * nchunks + k;
  const int n = lane & 15, g = lane >> 4;
  // a 64-channel token row is 16 bytes: lane groups 2 and 3 hold no codes
  const bool k_in = DD >= 128 || g < 2;
#pragma unroll
  for (int hf = 0; hf < Dm::NQ; ++hf) {
    const uint8_t *kc =
        a.k_codes + chunk * Dm::CB + Dm::KROW * slot_elem(n, 0) + 32 * hf + 8 * g;
#pragma unroll
    for (int t = 0; t < 8; ++t)  // token + 2 t
      r.k[hf][t] = k_in ? stream_load<u32x2>(kc + 2 * Dm::KROW * t) : u32x2{0u, 0u};
  }
  const uint8_t *vc = a.v_codes + chunk * Dm::CB + 32 * n + 8 * g;
#pragma unroll
  for (int ct = 0; ct < Dm::NCT; ++ct) r.v[ct] = stream_load<u32x2>(vc + 512 * ct);  // channel + 16 ct
  if constexpr (kTwoScales) {
    load_floats<Dm::CPL>(a.k_col + chunk * DD + Dm::CPL * lane, r.ck);
    load_floats<Dm::CPL>(a.v_col + chunk * DD + Dm::CPL * lane, r.cv);
  }
  const int64_t row = bg * (int64_t)a.capacity + (int64_t)k * T + 2 * lane;
  r.rk = stream_load<u32x2>(a.k_row + row);
  r.rv = stream_load<u32x2>(a.v_row + row);
}

template <int DD>
struct SplitState {
  float qv[Dims<DD>::NQ][8];  // query (rotated, scaled) at the channels of this lane's slot
  float acc[Dims<DD>::NCT];   // PV accumulators: head lane >> 4, channel 16 ct + (lane & 15)
  float m_run, l_run;
};

// The QK operand from this lane's 8 values x of head lane >> 4, slot
// lane & 15: per-head range scale, 4 fp8 terms written to rows 4 h + k of
// `rows`. Returns this lane's E8M0 row-scale byte for the operand it reads.
__device__ __forceinline__ int build_qk_operand(uint32_t (&rows)[16][OP_ROW], float (&x)[8],
                                                int lane) {
  const int n = lane & 15, h = lane >> 4;
  float mx = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) mx = fmaxf(mx, fabsf(x[j]));
  const int sig = range_exp8(group_max<16>(mx));
  const float sc = __builtin_ldexpf(1.f, sig);
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] *= sc;
  u32x2 t[4];
  fp8_terms<4>(x, t);
#pragma unroll
  for (int k = 0; k < 4; ++k) *reinterpret_cast<u32x2 *>(&rows[4 * h + k][2 * n]) = t[k];
  return row_scale_byte(sig, lane);
}

__device__ __forceinline__ u32x8 read_operand(const uint32_t (&rows)[16][OP_ROW], int lane) {
  const int n = lane & 15, h = lane >> 4;
  const u32x4 a0 = *reinterpret_cast<const u32x4 *>(&rows[n][8 * h]);
  const u32x4 a1 = *reinterpret_cast<const u32x4 *>(&rows[n][8 * h + 4]);
  return u32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
}

// kTwoScales = false: the column scales are taken as 1 (one-scale ablation);
// the QK operands (aq_fixed, sa_fixed) are then the same for every chunk.
template <int DD, bool kTwoScales>
__device__ __forceinline__ void process_chunk(DecSmem<DD> &sm, SplitState<DD> &st,
                                              const ChunkRegs<DD> &cur, int nvalid, int lane,
                                              const u32x8 (&aq_fixed)[Dims<DD>::NQ],
                                              const int (&sa_fixed)[Dims<DD>::NQ]) {
  using Dm = Dims<DD>;
  constexpr int NQ = Dm::NQ, NCT = Dm::NCT;
  const int n = lane & 15, h = lane >> 4;
  const int sb = slot_base(n);

  // ---- scales to LDS ----
  wave_lds_sync();  // after the previous chunk's readers
  {
    if constexpr (kTwoScales) {
#pragma unroll
      for (int i = 0; i < Dm::CPL; ++i) {
        const int e = Dm::CPL * lane + i;  // channel
        sm.ck[e >> 7][elem_pos(e & 127)] = cur.ck[i];
        sm.cv[cv_base(NCT, e & 15) + (e >> 4)] = cur.cv[i];
      }
    }
    const int e = 2 * lane;  // token; token e + 1 sits 8 further on
    const int pe = elem_pos(e);
    sm.rk[pe] = __uint_as_float(cur.rk[0]);
    sm.rk[pe + 8] = __uint_as_float(cur.rk[1]);
    sm.rv[pe] = __uint_as_float(cur.rv[0]);
    sm.rv[pe + 8] = __uint_as_float(cur.rv[1]);
  }
  wave_lds_sync();

  // ---- QK operands: head h, slot n: x = q * c_K * 2^sigma_h as 4 fp8 terms ----
  int sa_q[NQ];
  u32x8 aq[NQ];
#pragma unroll
  for (int hf = 0; hf < NQ; ++hf) {
    sa_q[hf] = sa_fixed[hf];
    aq[hf] = aq_fixed[hf];
  }
  if constexpr (kTwoScales) {
#pragma unroll
    for (int hf = 0; hf < NQ; ++hf) {
      const f32x4 c0 = *reinterpret_cast<const f32x4 *>(&sm.ck[hf][sb]);
      const f32x4 c1 = *reinterpret_cast<const f32x4 *>(&sm.ck[hf][sb + 4]);
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = st.qv[hf][j] * (j < 4 ? c0[j] : c1[j - 4]);
      sa_q[hf] = build_qk_operand(sm.aq[hf], x, lane);
    }
    wave_lds_sync();
#pragma unroll
    for (int hf = 0; hf < NQ; ++hf) aq[hf] = read_operand(sm.aq[hf], lane);
  }

  // ---- QK^T: 8 token tiles; the four terms of head h land in d[0..3] ----
  float s[8];
  {
    // all products are independent of each other's results except the
    // halves' accumulation: issue them back to back and sum the terms
    // afterwards, so the MFMA latency is paid once; the level offset of head
    // h (the same for every token) is added after the term sum
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 d[8];
#pragma unroll
    for (int tau = 0; tau < 8; ++tau) {
      d[tau] = mfma_f8f4(aq[0], code_operand(cur.k[0][tau]), zero, sa_q[0]);
      if constexpr (NQ == 2) d[tau] = mfma_f8f4(aq[1], code_operand(cur.k[1][tau]), d[tau], sa_q[1]);
    }
    f32x4 off = level_offset(aq[0], sa_q[0]);
    if constexpr (NQ == 2) off += level_offset(aq[1], sa_q[1]);
    const float off_h = (off[0] + off[1]) + (off[2] + off[3]);
#pragma unroll
    for (int tau = 0; tau < 8; ++tau)
      s[tau] = ((d[tau][0] + d[tau][1]) + (d[tau][2] + d[tau][3])) + off_h;
  }

  // ---- online softmax of head h over the tokens slot_elem(n, tau) ----
  {
    const f32x4 rk0 = *reinterpret_cast<const f32x4 *>(&sm.rk[sb]);
    const f32x4 rk1 = *reinterpret_cast<const f32x4 *>(&sm.rk[sb + 4]);
#pragma unroll
    for (int j = 0; j < 8; ++j) s[j] *= (j < 4 ? rk0[j] : rk1[j - 4]);
    if (nvalid < T) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (slot_elem(n, j) >= nvalid) s[j] = -INFINITY;
    }
    float mc = s[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mc = fmaxf(mc, s[j]);
    mc = group_max<16>(mc);
    // integer running max (log2 units): the probabilities of a chunk then
    // differ between split layouts only by powers of two, which the range
    // scale below absorbs exactly
    const float mn = fmaxf(st.m_run, ceilf(mc));
    const float al = exp2f(st.m_run - mn);  // 0 on the first chunk
    const f32x4 rv0 = *reinterpret_cast<const f32x4 *>(&sm.rv[sb]);
    const f32x4 rv1 = *reinterpret_cast<const f32x4 *>(&sm.rv[sb + 4]);
    float w[8];
    float ps = 0.f, mw = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = exp2f(s[j] - mn);
      ps += p;
      w[j] = p * (j < 4 ? rv0[j] : rv1[j - 4]);
    }
    if (nvalid < T) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (slot_elem(n, j) >= nvalid) w[j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) mw = fmaxf(mw, w[j]);
    const int sig = range_exp8(group_max<16>(mw));
    const float sc = __builtin_ldexpf(1.f, sig);
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] *= sc;
    u32x2 t[3];
    fp8_terms<3>(w, t);
#pragma unroll
    for (int k = 0; k < 3; ++k) *reinterpret_cast<u32x2 *>(&sm.ap[4 * h + k][2 * n]) = t[k];
    st.l_run = st.l_run * al + ps;
    st.m_run = mn;
    // the running max moves by whole powers of two and seldom: rescale only
    // when it moved for some head
    if (__builtin_amdgcn_ballot_w64(al != 1.f)) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) st.acc[ct] *= al;
    }
    const int sa_p = row_scale_byte(sig, lane);
    wave_lds_sync();

    // ---- PV: NCT channel tiles ----
    const u32x8 ap = read_operand(sm.ap, lane);
    float cvs[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) cvs[ct] = 1.f;
    if constexpr (kTwoScales) {
#pragma unroll
      for (int c4 = 0; c4 < NCT / 4; ++c4) {
        const f32x4 cv4 = *reinterpret_cast<const f32x4 *>(&sm.cv[cv_base(NCT, n) + 4 * c4]);
#pragma unroll
        for (int i = 0; i < 4; ++i) cvs[4 * c4 + i] = cv4[i];
      }
    }
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 d[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) d[ct] = mfma_f8f4(ap, code_operand(cur.v[ct]), zero, sa_p);
    const f32x4 off = level_offset(ap, sa_p);
    const float off_h = (off[0] + off[1]) + off[2];  // row 4 h + 3 is zero
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const float dv = ((d[ct][0] + d[ct][1]) + d[ct][2]) + off_h;
      if constexpr (kTwoScales)
        st.acc[ct] = fmaf(cvs[ct], dv, st.acc[ct]);
      else
        st.acc[ct] += dv;
    }
  }
}

// Last step for one query head, by one wave: lane l holds channels CPL l + i
// of the merged numerator x and every lane the denominator L;
// out = (x / L) H_DD / sqrt(DD), or x / L when the rotation is absorbed.
// The channel bits below CPL are the register index, the others lane bits:
// those butterfly stages are in registers, the rest exchange lanes.
template <int DD, bool kRotate>
__device__ __forceinline__ void finalize_head(float (&x)[Dims<DD>::CPL], float L, int lane,
                                              float *out) {
  constexpr int CPL = Dims<DD>::CPL;
  const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
  for (int i = 0; i < CPL; ++i) x[i] *= inv;
  if constexpr (kRotate) {
#pragma unroll
    for (int len = 1; len < CPL; len <<= 1)
#pragma unroll
      for (int i = 0; i < CPL; ++i)
        if ((i & len) == 0) {
          const float u = x[i], v = x[i + len];
          x[i] = u + v;
          x[i + len] = u - v;
        }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const bool upper = (lane & m) != 0;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const float p = lane_xor(x[i], m);
        x[i] = upper ? p - x[i] : x[i] + p;
      }
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i) x[i] *= inv_sqrt_head(DD);
  }
  if constexpr (CPL == 1) {
    out[lane] = x[0];
  } else if constexpr (CPL == 2) {
    *reinterpret_cast<f32x2 *>(out + 2 * lane) = f32x2{x[0], x[1]};
  } else {
    *reinterpret_cast<f32x4 *>(out + 4 * lane) = f32x4{x[0], x[1], x[2], x[3]};
  }
}

// Accesses to memory shared by the workgroups of one launch, coherent across
// the XCDs (agent scope; the device emits them with the system-coherence bit
// and no cache maintenance).
__device__ __forceinline__ void coherent_store(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void coherent_store2(float *p, f32x2 v) {
  __hip_atomic_store(reinterpret_cast<uint64_t *>(p), __builtin_bit_cast(uint64_t, v),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float *p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x2 coherent_load2(const float *p) {
  return __builtin_bit_cast(
      f32x2, __hip_atomic_load(reinterpret_cast<const uint64_t *>(p), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT));
}
// N consecutive floats (N = 1, 2 or 4; 8-byte aligned for N > 1)
template <int N>
__device__ __forceinline__ void coherent_store_n(float *p, const float (&v)[N]) {
  if constexpr (N == 1) {
    coherent_store(p, v[0]);
  } else {
#pragma unroll
    for (int i = 0; i < N; i += 2) coherent_store2(p + i, f32x2{v[i], v[i + 1]});
  }
}
template <int N>
__device__ __forceinline__ void coherent_load_n(const float *p, float (&v)[N]) {
  if constexpr (N == 1) {
    v[0] = coherent_load(p);
  } else {
#pragma unroll
    for (int i = 0; i < N; i += 2) {
      const f32x2 u = coherent_load2(p + i);
      v[i] = u[0];
      v[i + 1] = u[1];
    }
  }
}

// The four waves' results of a workgroup, merged in LDS.
template <int DD>
struct MergeSmem {
  float m[kDecWaves][HG];
  float l[kDecWaves][HG];
  alignas(16) float acc[kDecWaves][HG][DD];
  int last;
};

// Waves per SIMD the kernel's registers allow, by head size (the split count
// targets that many).
__host__ __device__ constexpr int decode_waves_per_simd(int dd) { return dd == 256 ? 2 : 3; }

// kRotate = false: the query comes rotated (rotation absorbed into the model's
// weights); kTwoScales = false: column scales taken as 1 (ablation).
//
// One workgroup = four waves = four consecutive splits of one (sequence,
// kv-head, head group). Split s of a row's n_wg * 4 takes the sequence's
// used chunks s, s + n_wg * 4, s + 2 n_wg * 4, ... (counts differ by at
// most one; splits past its length get none): the first chunk of a split
// does not depend on the length, so its loads go out before the length has
// arrived. After the chunk loop the four waves merge their
// (m, l, acc) in LDS, and wave h then carries head h0 + h: with one
// workgroup per row it writes the output directly; otherwise it writes the
// workgroup's partial, and the workgroup that finishes last (a counter per
// row in the workspace, reset by that workgroup) merges the row's partials
// and writes the output, so no second launch is needed.
template <int DD, bool kRotate, bool kTwoScales>
__global__ __launch_bounds__(64 * kDecWaves, decode_waves_per_simd(DD)) void decode_kernel(
    DecodeArgs a) {
  using Dm = Dims<DD>;
  constexpr int NQ = Dm::NQ, NCT = Dm::NCT, CPL = Dm::CPL;
  __shared__ DecSmem<DD> sms[kDecWaves];
  __shared__ MergeSmem<DD> mg;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  DecSmem<DD> &sm = sms[wv];
  const int G = a.q_heads / a.kv_heads;
  const int n_hg = (G + HG - 1) / HG;
  const int wgs = blockIdx.x % a.n_wg, hg = blockIdx.x / a.n_wg;
  const int g = blockIdx.y, b = blockIdx.z;
  const int h0 = hg * HG, nh = min(HG, G - h0);  // query heads g * G + h0 + [0, nh)
  const int nch = a.capacity / T;
  const int len = a.lens[b];
  const bool valid = len >= 1 && len <= a.capacity;
  const int used = valid ? (len + T - 1) / T : 0;
  const int n_split = a.n_wg * kDecWaves, split = wgs * kDecWaves + wv;
  const int64_t bg = (int64_t)b * a.kv_heads + g;
  const int64_t qh0 = (int64_t)b * a.q_heads + (int64_t)g * G + h0;
  const int64_t row = bg * n_hg + hg;  // counter index

  // ---- query: lane (slot n, head hl) keeps the channels of its slot in each
  // 128-channel half hf, 128 hf + slot_elem(n, j) = 128 hf + c0 + (n & 1) + 2 j,
  // and rotates them in registers: bits 1..3 of the channel index (j) and bit
  // 7 (hf) are in the lane, bits 0, 6, 4 and 5 are lane bits 0..3 of the
  // 16-lane row that holds the head (a 64-channel head has no bit 6: the
  // lanes of its upper slots hold zeros). Softmax scale, log2(e), 1/sqrt(DD)
  // and the 2 of the half-level code values are folded in. The query loads go
  // first and the first chunk's loads next, so that waiting for the query
  // leaves the chunk in flight during the set-up ----
  const int n_l = lane & 15, hl = lane >> 4;
  const int qc0 = slot_elem(n_l, 0) & ~1;  // 16-channel window holding the slot
  const bool q_in = qc0 < DD;
  // bf16 queries: the raw words first, then the first chunk, then the
  // conversion, so that the wait for the query leaves the chunk in flight
  // (vector-memory loads complete in order). Both loads are issued on every
  // path, from clamped in-bounds addresses, with the unused values dropped
  // afterwards: a load skipped on some path would leave the compiler unable
  // to count the loads issued after the query's, and it would wait for all
  // of them. fp32 queries (the small parity workload) are converted at once.
  const bool q_f32 = a.q_dtype == KVARN_DT_F32;
  const bool q_use = q_in && hl < nh;
  float qr[NQ][8];
  u32x4 qb[NQ][2];
#pragma unroll
  for (int hf = 0; hf < NQ; ++hf) {
    const int64_t qrow = (qh0 + min(hl, nh - 1)) * DD + 128 * hf + (q_in ? qc0 : 0);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) qr[hf][jj] = 0.f;
    qb[hf][0] = qb[hf][1] = u32x4{0u, 0u, 0u, 0u};
    if (!q_f32) {
      const u32x4 *qp = reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(a.q) + qrow);
      qb[hf][0] = qp[0];
      qb[hf][1] = qp[1];
    } else if (q_in) {
      const f32x4 *qf = reinterpret_cast<const f32x4 *>(static_cast<const float *>(a.q) + qrow);
      float qw[16];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const f32x4 v4 = qf[r];
        qw[4 * r] = v4[0]; qw[4 * r + 1] = v4[1]; qw[4 * r + 2] = v4[2]; qw[4 * r + 3] = v4[3];
      }
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)
        qr[hf][jj] = hl < nh ? ((n_l & 1) ? qw[2 * jj + 1] : qw[2 * jj]) : 0.f;
    }
  }
  ChunkRegs<DD> cur, nxt;
  // the split's first chunk, loaded before the sequence length is known;
  // a split past the cache's chunks loads the last one (in bounds) and
  // leaves it unused, as does one past the sequence's length
  load_chunk<DD, kTwoScales>(a, bg, nch, min(split, nch - 1), lane, cur);
  if (!q_f32) {
    // channel qc0 + 2 jj + (n & 1): bf16 element (n & 1) of word jj, moved
    // to the high half by a shift of 16 or 0
    const int q_sh = (n_l & 1) ? 0 : 16;
#pragma unroll
    for (int hf = 0; hf < NQ; ++hf)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const uint32_t w = (qb[hf][jj >> 2][jj & 3] << q_sh) & 0xFFFF0000u;
        qr[hf][jj] = q_use ? __uint_as_float(w) : 0.f;
      }
  }
  if constexpr (kRotate) {
#pragma unroll
    for (int hf = 0; hf < NQ; ++hf)
#pragma unroll
      for (int len2 = 1; len2 < 8; len2 <<= 1)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          if ((jj & len2) == 0) {
            const float u = qr[hf][jj], v = qr[hf][jj + len2];
            qr[hf][jj] = u + v;
            qr[hf][jj + len2] = u - v;
          }
    if constexpr (NQ == 2) {  // channel bit 7
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const float u = qr[0][jj], v = qr[1][jj];
        qr[0][jj] = u + v;
        qr[1][jj] = u - v;
      }
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
      if (DD == 64 && m == 2) continue;  // channel bit 6
      const bool upper = (n_l & m) != 0;
#pragma unroll
      for (int hf = 0; hf < NQ; ++hf)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const float p = lane_xor(qr[hf][jj], m);
          qr[hf][jj] = upper ? p - qr[hf][jj] : qr[hf][jj] + p;
        }
    }
  }
  for (int idx = lane; idx < 16 * OP_ROW; idx += 64) (&sm.ap[0][0])[idx] = 0u;
  if constexpr (DD == 64) {  // c_K of the slots past channel 64: never written, read as 0
    for (int idx = lane; idx < SLOT_ARRAY; idx += 64) sm.ck[0][idx] = 0.f;
  }
  SplitState<DD> st;
  {
    // the unscaled rotation's 1/sqrt(DD) applies only when it ran here
    const float qs = 2.f * a.scale * kLog2e * (kRotate ? inv_sqrt_head(DD) : 1.f);
#pragma unroll
    for (int hf = 0; hf < NQ; ++hf)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) st.qv[hf][jj] = qr[hf][jj] * qs;
  }
  // one scale: the QK operands do not change from chunk to chunk
  u32x8 aq_fixed[NQ];
  int sa_fixed[NQ];
#pragma unroll
  for (int hf = 0; hf < NQ; ++hf) {
    aq_fixed[hf] = u32x8{0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    sa_fixed[hf] = 127;
  }
  if constexpr (!kTwoScales) {
#pragma unroll
    for (int hf = 0; hf < NQ; ++hf) {
      float x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = st.qv[hf][j];
      sa_fixed[hf] = build_qk_operand(sm.aq[hf], x, lane);
    }
    wave_lds_sync();
#pragma unroll
    for (int hf = 0; hf < NQ; ++hf) aq_fixed[hf] = read_operand(sm.aq[hf], lane);
  }
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) st.acc[ct] = 0.f;
  st.m_run = -INFINITY;
  st.l_run = 0.f;

  // The first chunk has landed during the set-up. Waiting for it here, once,
  // keeps the loop's own waits on the chunk loaded one iteration ahead (a
  // load still pending on entry would make every iteration wait for the
  // loads it has just issued: the counter completes in order).
  __builtin_amdgcn_s_waitcnt(kVmcntZero);
  for (int k = split; k < used; k += n_split) {
    if (k + n_split < used) load_chunk<DD, kTwoScales>(a, bg, nch, k + n_split, lane, nxt);
    process_chunk<DD, kTwoScales>(sm, st, cur, min(len - k * T, T), lane, aq_fixed, sa_fixed);
    cur = nxt;
  }

  // ---- the four waves' (m, l, acc) meet in LDS; wave h then merges head h ----
  {
    const int h = lane >> 4, n = lane & 15;
    const float lsum = group_sum<16>(st.l_run);
    if (n == 0) {
      mg.m[wv][h] = st.m_run;
      mg.l[wv][h] = lsum;
    }
    // 2: the code operand carries c/2
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) mg.acc[wv][h][16 * ct + n] = 2.f * st.acc[ct];
  }
  __syncthreads();
  const int hh = wv;  // the head this wave merges (wave-uniform)
  float M = -INFINITY, L = 0.f;
  float x[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) x[i] = 0.f;
  if (hh < nh) {
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, mg.m[w][hh]);
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float mw = mg.m[w][hh];
      // the running maxima are whole numbers (log2 units): exact powers of two
      const float e = mw == -INFINITY ? 0.f : exp2f(mw - M);
      L = fmaf(e, mg.l[w][hh], L);
#pragma unroll
      for (int i = 0; i < CPL; ++i) x[i] = fmaf(e, mg.acc[w][hh][CPL * lane + i], x[i]);
    }
  }
  if (a.n_wg == 1) {
    if (hh < nh) finalize_head<DD, kRotate>(x, L, lane, a.out + (qh0 + hh) * DD);
    return;
  }
  // The workgroup that finishes its row last merges it. The partials and the
  // counter are the only memory shared between workgroups; they are written
  // and read coherently across the XCDs' separate L2 caches (agent-scope
  // accesses), each thread's partial stores complete before the count is
  // taken, and the last workgroup reads them after it. (A full agent-scope
  // fence would write back and invalidate the whole L2 of the XCD in every
  // workgroup, which costs more than the merge.)
  if (hh < nh) {
    float *pp = a.partial + ((qh0 + hh) * a.n_wg + wgs) * (2 + DD);
    if (lane == 0) {
      coherent_store(pp, M);
      coherent_store(pp + 1, L);
    }
    coherent_store_n<CPL>(pp + 2 + CPL * lane, x);
  }
  __builtin_amdgcn_s_waitcnt(kVmcntZero);
  __syncthreads();
  if (tid == 0)
    mg.last = __hip_atomic_fetch_add(a.counters + row, 1, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT) == a.n_wg - 1;
  __syncthreads();
  if (!mg.last) return;
  if (hh < nh) {
    // the row's partials in rounds of R, all loads of a round issued before
    // any is used, merged into a running (M, L, x) by log-sum-exp; R covers
    // the occupancy-derived workgroup count per row in one round (12 for head
    // sizes 64 and 128 on 256 CUs, 8 for 256), so the merge waits for memory
    // once
    const float *pp = a.partial + (qh0 + hh) * a.n_wg * (2 + DD);
    constexpr int R = DD == 256 ? 8 : 16;
    M = -INFINITY;
    L = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) x[i] = 0.f;
    for (int i0 = 0; i0 < a.n_wg; i0 += R) {
      float mi[R], li[R], xi[R][CPL];
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const float *pi = pp + (i0 + j) * (2 + DD);
        const bool in = i0 + j < a.n_wg;
        mi[j] = in ? coherent_load(pi) : -INFINITY;
        li[j] = in ? coherent_load(pi + 1) : 0.f;
        if (in) {
          coherent_load_n<CPL>(pi + 2 + CPL * lane, xi[j]);
        } else {
#pragma unroll
          for (int i = 0; i < CPL; ++i) xi[j][i] = 0.f;
        }
      }
      float mn = M;
#pragma unroll
      for (int j = 0; j < R; ++j) mn = fmaxf(mn, mi[j]);
      const float sc = M == -INFINITY ? 0.f : exp2f(M - mn);
      L *= sc;
#pragma unroll
      for (int i = 0; i < CPL; ++i) x[i] *= sc;
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const float e = mi[j] == -INFINITY ? 0.f : exp2f(mi[j] - mn);
        L = fmaf(e, li[j], L);
#pragma unroll
        for (int i = 0; i < CPL; ++i) x[i] = fmaf(e, xi[j][i], x[i]);
      }
      M = mn;
    }
    finalize_head<DD, kRotate>(x, L, lane, a.out + (qh0 + hh) * DD);
  }
  if (tid == 0)  // ready for the next call
    __hip_atomic_store(a.counters + row, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

// The split partials of kvarn_decode_attn_noalloc. In host code `scratch`
// names a host-side stand-in, not device memory: kernels get the address that
// hipGetSymbolAddress returns for the current device (each GPU holds its own
// copy), never the array's name.
static __device__ __align__(256) uint8_t scratch[KVARN_NOALLOC_SCRATCH_BYTES];

void *noalloc_scratch(hipError_t *err) {
  static std::mutex mu;
  static void *addr[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess && (dev < 0 || dev >= 64)) e = hipErrorInvalidDevice;
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    addr[dev] = p;
  }
  return addr[dev];
}

// Compute units of the current device, queried once per device (an MI355X
// has 256; that count is assumed if the query fails).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}
static int device_simds() { return 4 * device_cus(); }

// Workgroups per (sequence, kv-head, head group): about as many waves per
// SIMD as the kernel's registers allow for the head size, in one round
// (four-wave workgroups, one split per wave).
int decode_auto_wgs(int batch, int kv_heads, int q_heads, int capacity, int head_dim) {
  const int max_wg = decode_max_wgs(capacity);
  if (batch <= 0 || kv_heads <= 0 || q_heads <= 0 || max_wg <= 0) return 1;
  const int G = q_heads / kv_heads;
  const int64_t rows = (int64_t)batch * kv_heads * ((G + HG - 1) / HG);
  const int64_t target = (int64_t)decode_waves_per_simd(head_dim) * device_simds() / kDecWaves;
  int64_t s = (target + rows / 2) / rows;
  if (s > max_wg) s = max_wg;
  if (s < 1) s = 1;
  return (int)s;
}

template <int DD>
static hipError_t launch_decode_dd(const DecodeArgs &a, hipStream_t s) {
  if (a.batch == 0 || a.q_heads == 0) return hipSuccess;
  const int G = a.q_heads / a.kv_heads;
  const int n_hg = (G + HG - 1) / HG;
  const dim3 grid(a.n_wg * n_hg, a.kv_heads, a.batch), block(64 * kDecWaves);
  const bool rot = !(a.flags & KVARN_FLAG_NO_ROTATE), two = !(a.flags & KVARN_FLAG_ONE_SCALE);
  if (rot && two)
    hipLaunchKernelGGL((decode_kernel<DD, true, true>), grid, block, 0, s, a);
  else if (rot)
    hipLaunchKernelGGL((decode_kernel<DD, true, false>), grid, block, 0, s, a);
  else if (two)
    hipLaunchKernelGGL((decode_kernel<DD, false, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((decode_kernel<DD, false, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
  switch (a.head_dim) {
    case 64: return launch_decode_dd<64>(a, s);
    case 256: return launch_decode_dd<256>(a, s);
    default: return launch_decode_dd<128>(a, s);
  }
}

}  // namespace kvarn
