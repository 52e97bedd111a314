/*
 * kvarn.h -- C ABI of libkvarn.so, the MI355X (gfx950) KVarN KV-cache
 * quantizer and the 2-bit decode attention that reads its cache.
 *
 * The method (arXiv 2606.03458, "KVarN: Variance-Normalized KV-Cache
 * Quantization Mitigates Error Accumulation in Reasoning Tasks"; abstract as
 * carried by the codewithpapers.app record; rndamp.com article on KVarN,
 * sections "How It Works" and "Numbers"): each per-head K or V block is
 * rotated by a Hadamard transform along the channel dimension, balanced on
 * both axes by an iterative dual scaling, and stored at 2 bits; the
 * dequantization applies both scales inside the attention kernel. The
 * quantizer needs no calibration data, so no call below takes any.
 *
 * Conventions shared by every call
 *  - Pointers marked (device) are HIP device pointers; (host) are host
 *    pointers read synchronously before the call returns.
 *  - The caller allocates and owns every buffer. The library allocates no
 *    device memory, keeps no state between calls and is reentrant across
 *    streams (two calls that write the same cache on different streams race).
 *  - `stream` is a hipStream_t (NULL = default stream). Every call only
 *    enqueues work and returns; the library never synchronizes. Device faults
 *    surface at the caller's next synchronization.
 *  - Arguments are validated on the host before any HIP call. On a validation
 *    error the call returns a negative kvarn_status and enqueues nothing.
 *    A failed launch returns KVARN_ERR_HIP.
 *  - The chunk (block) length is 128 tokens. head_dim is 128, 64 or 256 (a
 *    field of the cache descriptor). The block quantizer and decode run the
 *    same kernels for every head size; the one-token append and the token
 *    error run simpler kernels for 64 and 256 that compute the same
 *    quantities.
 */
#ifndef KVARN_H
#define KVARN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    KVARN_HEAD_DIM = 128,   /* channels per head (power of two for the rotation) */
    KVARN_CHUNK = 128,      /* tokens per quantization block */
    KVARN_CHUNK_BYTES = 4096, /* packed 2-bit codes of one 128 x 128 block */
    KVARN_DECODE_WAVES = 4    /* decode splits per workgroup */
};

typedef enum {
    KVARN_OK = 0,
    KVARN_ERR_NULL = -1,      /* a required pointer is NULL */
    KVARN_ERR_SHAPE = -2,     /* a size, stride or count is out of range */
    KVARN_ERR_ALIGN = -3,     /* a pointer or stride breaks 16-byte alignment */
    KVARN_ERR_DTYPE = -4,     /* unknown dtype or cache kind */
    KVARN_ERR_CAPACITY = -5,  /* tokens + token_offset exceed the cache capacity */
    KVARN_ERR_WORKSPACE = -6, /* workspace smaller than kvarn_decode_workspace_bytes */
    KVARN_ERR_HIP = -7,       /* a HIP launch or query failed */
    KVARN_ERR_FLAGS = -8      /* a flag bit this call does not know */
} kvarn_status;

typedef enum { KVARN_DT_BF16 = 0, KVARN_DT_F32 = 1 } kvarn_dtype;

/*
 * Flags of the *_ex calls (0 = the method as specified).
 *
 * KVARN_FLAG_NO_ROTATE  the rotation is absorbed into the model's weights
 *     (rndamp article on KVarN, "How It Works", item 1: the Hadamard transform
 *     can be folded into existing weights): quantize and append take K/V that
 *     are already rotated (x . H_D / sqrt(D), D = head_dim) and skip the
 *     rotation; decode takes the rotated query q . H_D / sqrt(D) and returns
 *     the output in the rotated basis (out . H_D / sqrt(D) is the output in
 *     the original basis).
 * KVARN_FLAG_ONE_SCALE  (decode only) ablation of the second scale: the
 *     column scales are treated as 1 and not read ("Numbers": two scales
 *     instead of one; the cost of fusing the second one is what this
 *     measures). Meaningful on caches quantized with iters = 0, whose column
 *     scales are 1; on other caches it computes attention over y_hat / c.
 */
enum {
    KVARN_FLAG_NO_ROTATE = 1u << 0,
    KVARN_FLAG_ONE_SCALE = 1u << 1
};

/* K caches store codes token-major, V caches channel-major (see below). */
typedef enum { KVARN_K = 0, KVARN_V = 1 } kvarn_kind;

/*
 * One K or V cache of one layer. All three arrays are (device) memory owned
 * by the caller; capacity % 128 == 0; every pointer 16-byte aligned. D is
 * head_dim (0 stands for 128; 64, 128 and 256 are supported).
 *
 * codes      [batch][kv_heads][capacity/128][32 D] bytes (4096 for D = 128).
 *            Four 2-bit codes per byte, lowest bits first. Within a
 *            128-token chunk:
 *              K: token t owns bytes [D/4 t, D/4 (t + 1)); channel j sits in
 *                 byte D/4 t + j/4 at bits 2 (j % 4);
 *              V: channel j owns bytes [32 j, 32 j + 32); token t sits in
 *                 byte 32 j + t/4 at bits 2 (t % 4).
 *            Code q in {0,1,2,3} stands for the level (q - 1.5).
 * row_scale  [batch][kv_heads][capacity] fp32: per-token scale r'_t.
 * col_scale  [batch][kv_heads][capacity/128][D] fp32: per-chunk, per-channel
 *            scale c_j.
 * The stored value is reconstructed in the rotated basis as
 *   y_hat[t][j] = (code[t][j] - 1.5) * row_scale[t] * col_scale[t/128][j]
 * and in the original basis as y_hat . H_D / sqrt(D), H_D the Sylvester-order
 * Hadamard matrix (the "two scales" of the rndamp article's "Numbers"
 * section). The calls below are written for D = 128; for another D read D
 * wherever 128 stands for the channel count.
 */
typedef struct {
    uint8_t *codes;
    float *row_scale;
    float *col_scale;
    int32_t batch;
    int32_t kv_heads;
    int32_t capacity;
    int32_t kind;     /* kvarn_kind */
    int32_t head_dim; /* D: 0 (= 128), 64, 128 or 256 */
} kvarn_cache;

/*
 * kvarn_quantize -- quantize whole 128-token chunks of K or V into a cache:
 * rotate each token along the channels, balance the block's token and
 * channel scales, store 2-bit codes (abstract, codewithpapers.app record;
 * rndamp article on KVarN, "How It Works", items 1 and 2).
 *
 * For every (b, h) and every chunk of x's tokens [0, tokens):
 *   y  = x_chunk . H_D / sqrt(D)                     (rotation per token)
 *   c  = 1; repeat `iters` times:                    (dual scaling)
 *          r_i^2 = mean_j y_ij^2 / c_j^2 ;  c_j^2 = mean_i y_ij^2 / r_i^2
 *   r'_i = max_j |y_ij| / c_j / 2                    (per-token range step)
 *   code = min(3, floor(y_ij / (r'_i c_j) + 2))      (4-level mid-rise grid)
 * and store codes, r' and c at cache slots [token_offset, token_offset+tokens).
 * A zero token row stores r' = 0 and code 2; a zero column keeps c_j = 1.
 * Non-finite input gives unspecified codes and scales for its chunk.
 * The arithmetic is fp32 on the unscaled rotation (y sqrt(D)): a token's
 * energy D sum_j x_j^2 must stay below 2^127 (|x| below about 2^53). Over
 * that range, scaling x by 2^k scales r' by exactly 2^k and leaves codes and c
 * bit-identical, as long as the squared rotated values stay normal fp32
 * numbers. A nonzero token whose energy is below 2^-126 is weighted as if it
 * were 2^-126.
 *
 * x          (device) input, dtype `dtype`, logical shape
 *            [dst->batch][dst->kv_heads][tokens][D], element (b,h,t,j) at
 *            x + b*stride_b + h*stride_h + t*stride_t + j (strides in elements,
 *            channels contiguous). x must be 16-byte aligned and every stride
 *            a multiple of 16 bytes.
 * tokens, token_offset  multiples of 128; token_offset + tokens <= capacity.
 *            tokens == 0 is a no-op (x may then be NULL).
 * iters      balancing iterations, 0..64 (the spec default is 4; 0 keeps c = 1,
 *            i.e. rotation and per-token step only).
 * dst        (host) cache descriptor; its arrays are written, nothing is read.
 */
int kvarn_quantize(const void *x, int32_t dtype, int64_t stride_b,
                   int64_t stride_h, int64_t stride_t, int32_t tokens,
                   int32_t token_offset, int32_t iters, const kvarn_cache *dst,
                   void *stream);

/* kvarn_quantize with flags: KVARN_FLAG_NO_ROTATE only (other bits give
 * KVARN_ERR_FLAGS). With it, x is taken as already rotated and the row scale
 * is r' = max_j |x_ij / c_j| / 2 of x itself. */
int kvarn_quantize_ex(const void *x, int32_t dtype, int64_t stride_b,
                      int64_t stride_h, int64_t stride_t, int32_t tokens,
                      int32_t token_offset, int32_t iters, uint32_t flags,
                      const kvarn_cache *dst, void *stream);

/*
 * kvarn_append -- quantize one new token per sequence into an existing cache
 * (rndamp article, "The Problem": during decoding the cache grows one token
 * per step and errors carry from step to step).
 *
 * For each (b, h): pos = positions[b]; skipped when pos is outside
 * [0, capacity). chunk k = pos / 128. When pos % 128 == 0 the chunk is opened:
 * its column scales are copied from chunk k-1 of the same (b, h), or set to 1
 * for k == 0. The token is rotated and coded against chunk k's column scales
 * with its own range step r' = max_j |y_j| / c_j / 2, exactly as in
 * kvarn_quantize; the chunk is not re-balanced. In a V cache, a token with
 * pos % 4 == 0 rewrites its whole byte (the three later token slots of that
 * byte become code 0); other tokens replace only their own 2 bits.
 *
 * x          (device) [batch][kv_heads][D], dtype `dtype`, contiguous,
 *            16-byte aligned.
 * positions  (device) int32 [batch].
 */
int kvarn_append(const void *x, int32_t dtype, const int32_t *positions,
                 const kvarn_cache *dst, void *stream);

/* kvarn_append with flags: KVARN_FLAG_NO_ROTATE only. */
int kvarn_append_ex(const void *x, int32_t dtype, const int32_t *positions,
                    uint32_t flags, const kvarn_cache *dst, void *stream);

/*
 * kvarn_append_kv -- one decoding step's new K and V tokens in one launch
 * (rndamp article, "The Problem": both caches grow by one token per step).
 * The result is exactly that of kvarn_append_ex(xk, ..., k) followed by
 * kvarn_append_ex(xv, ..., v): the two caches are disjoint, and each (b, h)
 * of each cache is coded by one wave as there.
 *
 * xk, xv     (device) [batch][kv_heads][D] each, dtype `dtype`, contiguous,
 *            16-byte aligned.
 * positions  (device) int32 [batch], shared by both caches.
 * flags      KVARN_FLAG_NO_ROTATE only.
 * k, v       a K cache and a V cache of the same batch, kv_heads, capacity
 *            and head size (else KVARN_ERR_DTYPE or KVARN_ERR_SHAPE).
 * Errors as for kvarn_append; on error nothing is enqueued.
 */
int kvarn_append_kv(const void *xk, const void *xv, int32_t dtype,
                    const int32_t *positions, uint32_t flags,
                    const kvarn_cache *k, const kvarn_cache *v, void *stream);

/*
 * kvarn_append_rebalance -- append with re-balancing at chunk close, the
 * alternative to kvarn_append's frozen column scales (the pages do not fix
 * how a new token enters the cache; the rndamp article's "The Problem" only
 * says errors carry from one decoding step into the next).
 *
 * Each token is appended exactly as by kvarn_append_ex (coded at once against
 * the open chunk's column scales) and is also stored, as given, in `window`
 * at slot pos % 128 of its (b, h). When the token fills its chunk
 * (pos % 128 == 127), that chunk is quantized again from the window with the
 * full dual scaling, exactly as kvarn_quantize_ex would quantize those 128
 * tokens with `iters` iterations, replacing the chunk's codes, row scales and
 * column scales. Decode reads the cache as usual.
 *
 * window     (device) [batch][kv_heads][128][D] of `dtype`, 16-byte
 *            aligned, caller-owned and kept between calls (no need to clear
 *            it). A chunk is re-quantized correctly only if all its 128
 *            tokens were appended through this call.
 * iters      0..64, as for kvarn_quantize.
 * flags      KVARN_FLAG_NO_ROTATE only.
 * Other arguments as for kvarn_append. Two kernels are enqueued on `stream`.
 */
int kvarn_append_rebalance(const void *x, int32_t dtype,
                           const int32_t *positions, void *window,
                           int32_t iters, uint32_t flags,
                           const kvarn_cache *dst, void *stream);

/*
 * kvarn_decode_workspace_bytes -- (host only) bytes of device workspace that
 * kvarn_decode_attn needs for these sizes: one int32 counter per (sequence,
 * query head) rounded up to 256 bytes, then the split-KV partial results of
 * the largest split count the capacity allows. Returns 0 for invalid sizes.
 */
size_t kvarn_decode_workspace_bytes(int32_t batch, int32_t q_heads,
                                    int32_t capacity);
/* The same for caches of head size head_dim (64, 128 or 256); 0 for invalid
 * sizes. kvarn_decode_workspace_bytes is this with head_dim 128. */
size_t kvarn_decode_workspace_bytes_ex(int32_t batch, int32_t q_heads,
                                       int32_t capacity, int32_t head_dim);

/*
 * kvarn_decode_attn -- one decoding step of grouped-query attention over the
 * 2-bit cache, dequantizing on the fly with both scales fused ("Numbers":
 * the second scale is folded into the dequantization kernel).
 *
 * For each sequence b and query head h (kv-head g = h / (q_heads/kv_heads)):
 *   s_t = softmax_scale * < q[b][h], K_hat[b][g][t] >   for t in [0, L_b)
 *   out[b][h] = sum_t softmax(s)_t * V_hat[b][g][t]
 * with K_hat, V_hat the caches' reconstructions in the original basis
 * (L_b = seq_lens[b]). A sequence with L_b outside [1, capacity] gets a zero
 * output row.
 *
 * q          (device) [batch][q_heads][D], dtype q_dtype, contiguous,
 *            unrotated (post positional encoding).
 * k, v       (host) descriptors of the K and V caches of one layer: same
 *            batch, kv_heads, capacity and head_dim; kinds KVARN_K and KVARN_V.
 * seq_lens   (device) int32 [batch].
 * out        (device) fp32 [batch][q_heads][D], original basis.
 * n_split    number of token splits per (b, kv-head); 0 lets the library
 *            choose. Rounded up to a multiple of KVARN_DECODE_WAVES (the
 *            splits of one workgroup) and clamped to [KVARN_DECODE_WAVES,
 *            capacity/128 rounded up to that multiple]. Each sequence's used
 *            chunks are dealt round-robin over the splits (counts differ
 *            by at most one).
 * workspace  (device) at least kvarn_decode_workspace_bytes_ex(batch,
 *            q_heads, capacity, head_dim) bytes, 16-byte aligned. Its leading counter bytes must
 *            be zero before the first call (a zero-filled allocation); every
 *            call leaves them zero again, the rest is scratch. Calls that
 *            share a workspace must not overlap in time.
 */
int kvarn_decode_attn(const void *q, int32_t q_dtype, int32_t q_heads,
                      const kvarn_cache *k, const kvarn_cache *v,
                      const int32_t *seq_lens, float softmax_scale, float *out,
                      int32_t n_split, void *workspace, size_t workspace_bytes,
                      void *stream);

/* kvarn_decode_attn with flags: KVARN_FLAG_NO_ROTATE, KVARN_FLAG_ONE_SCALE. */
int kvarn_decode_attn_ex(const void *q, int32_t q_dtype, int32_t q_heads,
                         const kvarn_cache *k, const kvarn_cache *v,
                         const int32_t *seq_lens, float softmax_scale,
                         uint32_t flags, float *out, int32_t n_split,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * kvarn_decode_attn_noalloc -- kvarn_decode_attn_ex without a workspace
 * argument and without any allocation, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc. The split partial results go to a device array
 * inside the library, KVARN_NOALLOC_SCRATCH_BYTES per GPU, held by each GPU
 * the library runs on until the process ends.
 *
 * Same arguments, results and kernels as kvarn_decode_attn_ex. A call uses
 * the counters (batch * q_heads * 4 bytes rounded up to 256) and the
 * partials of its workgroups, batch * q_heads * W * (2 + D) * 4 bytes with
 * W = n_split / KVARN_DECODE_WAVES rounded up (clamped as for
 * kvarn_decode_attn) or the library's choice for n_split == 0; a call that
 * needs more than KVARN_NOALLOC_SCRATCH_BYTES returns KVARN_ERR_WORKSPACE and
 * enqueues nothing. The array starts zeroed and every call leaves its
 * counters zero. The work runs on the current device, which must be the
 * device of `stream`. Every call on one GPU shares that GPU's array: two
 * calls that may overlap in time on one GPU (different streams, different
 * host threads) race and must be ordered by the caller.
 */
enum { KVARN_NOALLOC_SCRATCH_BYTES = 16 << 20 };
int kvarn_decode_attn_noalloc(const void *q, int32_t q_dtype, int32_t q_heads,
                              const kvarn_cache *k, const kvarn_cache *v,
                              const int32_t *seq_lens, float softmax_scale,
                              uint32_t flags, float *out, int32_t n_split,
                              void *stream);

/*
 * kvarn_token_error -- per-token magnitude and direction of the cache's
 * reconstruction against the original K or V (rndamp article on KVarN,
 * "The Problem": the error of K is one of token magnitude rather than of
 * direction; "How It Works", closing paragraph: the method minimizes the
 * magnitude component). A diagnostic; it reads the cache and writes nothing
 * else.
 *
 * For every (b, h) and i in [0, tokens), cache slot t = token_offset + i:
 *   ratio[b][h][i]  = ||x_hat_t|| / ||x_t||
 *   cosine[b][h][i] = <x_hat_t, x_t> / (||x_hat_t|| ||x_t||)
 * with x_t = x's token i and x_hat_t the cache's reconstruction of slot t
 * (both in the original basis; the rotation preserves both numbers, so they
 * are computed in the rotated one). Degenerate tokens: both zero -> (1, 1);
 * x_t zero only -> (+inf, 0); x_hat_t zero only -> (0, 0). Sums in fp32.
 *
 * x          (device) as for kvarn_quantize: [batch][kv_heads][tokens][D],
 *            dtype `dtype`, strides in elements, 16-byte aligned pointer and
 *            strides. With KVARN_FLAG_NO_ROTATE x is taken as already rotated.
 * tokens     any count >= 0 (0 is a no-op); token_offset >= 0;
 *            token_offset + tokens <= capacity.
 * cache      (host) descriptor, read only.
 * ratio, cosine  (device) fp32 [batch][kv_heads][tokens], 4-byte aligned,
 *            written.
 * flags      KVARN_FLAG_NO_ROTATE only.
 */
int kvarn_token_error(const void *x, int32_t dtype, int64_t stride_b,
                      int64_t stride_h, int64_t stride_t, int32_t tokens,
                      int32_t token_offset, uint32_t flags,
                      const kvarn_cache *cache, float *ratio, float *cosine,
                      void *stream);

/* kvarn_status_string -- (host only) static text for a kvarn_status. */
const char *kvarn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* KVARN_H */
