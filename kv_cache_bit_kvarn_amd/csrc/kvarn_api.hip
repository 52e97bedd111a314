// extern "C" entry points of libkvarn.so: host-side validation, grid sizing,
// launch. Every check runs before any HIP call; a failed check enqueues
// nothing. The library allocates nothing and never synchronizes.
#include <limits.h>

#include "kvarn_diag.h"

using namespace kvarn;

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// head_dim of a cache (0 stands for 128)
int cache_dim(const kvarn_cache *c) { return c->head_dim == 0 ? D : c->head_dim; }
bool dim_ok(int d) { return d == 64 || d == 128 || d == 256; }

int check_cache(const kvarn_cache *c) {
  if (!c) return KVARN_ERR_NULL;
  if (!c->codes || !c->row_scale || !c->col_scale) return KVARN_ERR_NULL;
  if (c->kind != KVARN_K && c->kind != KVARN_V) return KVARN_ERR_DTYPE;
  if (c->batch < 0 || c->kv_heads < 0 || c->capacity < 0 || c->capacity % T != 0)
    return KVARN_ERR_SHAPE;
  if (!dim_ok(cache_dim(c))) return KVARN_ERR_SHAPE;
  if (!aligned16(c->codes) || !aligned16(c->row_scale) || !aligned16(c->col_scale))
    return KVARN_ERR_ALIGN;
  return KVARN_OK;
}

int dtype_size(int32_t dtype) {
  if (dtype == KVARN_DT_BF16) return 2;
  if (dtype == KVARN_DT_F32) return 4;
  return 0;
}

int from_hip(hipError_t e) { return e == hipSuccess ? KVARN_OK : KVARN_ERR_HIP; }

hipError_t run_decode(const DecodeArgs &a, hipStream_t s) { return launch_decode(a, s); }

// Checks shared by the decode entry points (everything but the workspace).
int check_decode(const void *q, int32_t q_dtype, int32_t q_heads, const kvarn_cache *k,
                 const kvarn_cache *v, const int32_t *seq_lens, float softmax_scale,
                 uint32_t flags, const float *out, int32_t n_split) {
  if (flags & ~(uint32_t)(KVARN_FLAG_NO_ROTATE | KVARN_FLAG_ONE_SCALE)) return KVARN_ERR_FLAGS;
  if (!q || !seq_lens || !out) return KVARN_ERR_NULL;
  int st = check_cache(k);
  if (st != KVARN_OK) return st;
  st = check_cache(v);
  if (st != KVARN_OK) return st;
  if (k->kind != KVARN_K || v->kind != KVARN_V) return KVARN_ERR_DTYPE;
  if (!dtype_size(q_dtype)) return KVARN_ERR_DTYPE;
  if (k->batch != v->batch || k->kv_heads != v->kv_heads || k->capacity != v->capacity ||
      cache_dim(k) != cache_dim(v))
    return KVARN_ERR_SHAPE;
  if (q_heads <= 0 || k->kv_heads <= 0 || q_heads % k->kv_heads) return KVARN_ERR_SHAPE;
  if (q_heads / k->kv_heads > GQA_MAX) return KVARN_ERR_SHAPE;
  if (k->capacity <= 0 || k->batch > 65535 || k->kv_heads > 65535 || q_heads > 65535)
    return KVARN_ERR_SHAPE;
  if (!(softmax_scale == softmax_scale)) return KVARN_ERR_SHAPE;  // NaN
  if (!aligned16(q) || !aligned16(out)) return KVARN_ERR_ALIGN;
  if (n_split < 0) return KVARN_ERR_SHAPE;
  return KVARN_OK;
}

// Workgroups per row of a call with valid arguments (HIP may be queried):
// n_split splits rounded up to whole workgroups, at most one split per chunk
// of capacity (rounded up to a workgroup), or the library's choice for 0.
int decode_wgs(int32_t q_heads, const kvarn_cache *k, int32_t n_split) {
  const int max_wg = decode_max_wgs(k->capacity);
  int nw = n_split == 0 ? decode_auto_wgs(k->batch, k->kv_heads, q_heads, k->capacity,
                                                         cache_dim(k))
                        : (int)(((int64_t)n_split + KVARN_DECODE_WAVES - 1) / KVARN_DECODE_WAVES);
  if (nw > max_wg) nw = max_wg;
  if (nw < 1) nw = 1;
  return nw;
}

DecodeArgs decode_args(const void *q, int32_t q_dtype, int32_t q_heads, const kvarn_cache *k,
                       const kvarn_cache *v, const int32_t *seq_lens, float softmax_scale,
                       uint32_t flags, float *out, int n_wg, void *workspace) {
  DecodeArgs a;
  a.q = q;
  a.q_dtype = q_dtype;
  a.batch = k->batch;
  a.q_heads = q_heads;
  a.kv_heads = k->kv_heads;
  a.capacity = k->capacity;
  a.head_dim = cache_dim(k);
  a.n_wg = n_wg;
  a.k_codes = k->codes;
  a.v_codes = v->codes;
  a.k_row = k->row_scale;
  a.k_col = k->col_scale;
  a.v_row = v->row_scale;
  a.v_col = v->col_scale;
  a.lens = seq_lens;
  a.scale = softmax_scale;
  a.flags = flags;
  a.out = out;
  a.counters = static_cast<int32_t *>(workspace);
  a.partial = reinterpret_cast<float *>(static_cast<char *>(workspace) +
                                        decode_counter_bytes(k->batch, q_heads));
  return a;
}


}  // namespace

extern "C" {

int kvarn_quantize_ex(const void *x, int32_t dtype, int64_t stride_b, int64_t stride_h,
                      int64_t stride_t, int32_t tokens, int32_t token_offset, int32_t iters,
                      uint32_t flags, const kvarn_cache *dst, void *stream) {
  if (flags & ~(uint32_t)KVARN_FLAG_NO_ROTATE) return KVARN_ERR_FLAGS;
  int st = check_cache(dst);
  if (st != KVARN_OK) return st;
  if (tokens == 0) return KVARN_OK;  // nothing to read or write; x may be NULL
  if (!x) return KVARN_ERR_NULL;
  const int esz = dtype_size(dtype);
  if (!esz) return KVARN_ERR_DTYPE;
  if (tokens < 0 || token_offset < 0 || tokens % T || token_offset % T) return KVARN_ERR_SHAPE;
  if (iters < 0 || iters > 64) return KVARN_ERR_SHAPE;
  if (stride_b < 0 || stride_h < 0 || stride_t < cache_dim(dst)) return KVARN_ERR_SHAPE;
  if ((int64_t)tokens + token_offset > dst->capacity) return KVARN_ERR_CAPACITY;
  if (!aligned16(x) || (stride_b * esz) % 16 || (stride_h * esz) % 16 || (stride_t * esz) % 16)
    return KVARN_ERR_ALIGN;
  const int64_t blocks = (int64_t)dst->batch * dst->kv_heads * (tokens / T);
  if (blocks > INT_MAX) return KVARN_ERR_SHAPE;
  if (blocks == 0) return KVARN_OK;
  QuantArgs a;
  a.x = x;
  a.dtype = dtype;
  a.sb = stride_b;
  a.sh = stride_h;
  a.st = stride_t;
  a.batch = dst->batch;
  a.heads = dst->kv_heads;
  a.chunks = tokens / T;
  a.chunk0 = token_offset / T;
  a.nblocks = (uint32_t)blocks;
  a.div_chunks = make_fastdiv((uint32_t)a.chunks);
  a.div_heads = make_fastdiv((uint32_t)a.heads);
  a.iters = iters;
  a.flags = flags;
  a.capacity = dst->capacity;
  a.kind = dst->kind;
  a.codes = dst->codes;
  a.row_scale = dst->row_scale;
  a.col_scale = dst->col_scale;
  a.pos = nullptr;
  a.head_dim = cache_dim(dst);
  return from_hip(launch_quantize(a, static_cast<hipStream_t>(stream)));
}

int kvarn_quantize(const void *x, int32_t dtype, int64_t stride_b, int64_t stride_h,
                   int64_t stride_t, int32_t tokens, int32_t token_offset, int32_t iters,
                   const kvarn_cache *dst, void *stream) {
  return kvarn_quantize_ex(x, dtype, stride_b, stride_h, stride_t, tokens, token_offset, iters,
                           0u, dst, stream);
}

int kvarn_append_ex(const void *x, int32_t dtype, const int32_t *positions, uint32_t flags,
                    const kvarn_cache *dst, void *stream) {
  if (flags & ~(uint32_t)KVARN_FLAG_NO_ROTATE) return KVARN_ERR_FLAGS;
  if (!x || !positions) return KVARN_ERR_NULL;
  int st = check_cache(dst);
  if (st != KVARN_OK) return st;
  if (!dtype_size(dtype)) return KVARN_ERR_DTYPE;
  if (!aligned16(x)) return KVARN_ERR_ALIGN;
  if ((int64_t)dst->batch * dst->kv_heads > INT_MAX) return KVARN_ERR_SHAPE;
  if (dst->batch == 0 || dst->kv_heads == 0 || dst->capacity == 0) return KVARN_OK;
  AppendArgs a;
  a.x = x;
  a.dtype = dtype;
  a.pos = positions;
  a.batch = dst->batch;
  a.heads = dst->kv_heads;
  a.capacity = dst->capacity;
  a.kind = dst->kind;
  a.flags = flags;
  a.codes = dst->codes;
  a.row_scale = dst->row_scale;
  a.col_scale = dst->col_scale;
  a.window = nullptr;
  a.head_dim = cache_dim(dst);
  return from_hip(launch_append(a, static_cast<hipStream_t>(stream)));
}

int kvarn_append(const void *x, int32_t dtype, const int32_t *positions,
                 const kvarn_cache *dst, void *stream) {
  return kvarn_append_ex(x, dtype, positions, 0u, dst, stream);
}

int kvarn_append_kv(const void *xk, const void *xv, int32_t dtype, const int32_t *positions,
                    uint32_t flags, const kvarn_cache *k, const kvarn_cache *v, void *stream) {
  if (flags & ~(uint32_t)KVARN_FLAG_NO_ROTATE) return KVARN_ERR_FLAGS;
  if (!xk || !xv || !positions) return KVARN_ERR_NULL;
  int st = check_cache(k);
  if (st != KVARN_OK) return st;
  st = check_cache(v);
  if (st != KVARN_OK) return st;
  if (k->kind != KVARN_K || v->kind != KVARN_V) return KVARN_ERR_DTYPE;
  if (!dtype_size(dtype)) return KVARN_ERR_DTYPE;
  if (k->batch != v->batch || k->kv_heads != v->kv_heads || k->capacity != v->capacity ||
      cache_dim(k) != cache_dim(v))
    return KVARN_ERR_SHAPE;
  if (!aligned16(xk) || !aligned16(xv)) return KVARN_ERR_ALIGN;
  if ((int64_t)k->batch * k->kv_heads > INT_MAX) return KVARN_ERR_SHAPE;
  if (k->batch == 0 || k->kv_heads == 0 || k->capacity == 0) return KVARN_OK;
  AppendArgs a[2];
  const kvarn_cache *c[2] = {k, v};
  const void *x[2] = {xk, xv};
  for (int i = 0; i < 2; ++i) {
    a[i].x = x[i];
    a[i].dtype = dtype;
    a[i].pos = positions;
    a[i].batch = c[i]->batch;
    a[i].heads = c[i]->kv_heads;
    a[i].capacity = c[i]->capacity;
    a[i].kind = c[i]->kind;
    a[i].flags = flags;
    a[i].codes = c[i]->codes;
    a[i].row_scale = c[i]->row_scale;
    a[i].col_scale = c[i]->col_scale;
    a[i].window = nullptr;
    a[i].head_dim = cache_dim(c[i]);
  }
  return from_hip(launch_append_kv(a[0], a[1], static_cast<hipStream_t>(stream)));
}

int kvarn_append_rebalance(const void *x, int32_t dtype, const int32_t *positions, void *window,
                           int32_t iters, uint32_t flags, const kvarn_cache *dst, void *stream) {
  if (flags & ~(uint32_t)KVARN_FLAG_NO_ROTATE) return KVARN_ERR_FLAGS;
  if (!x || !positions || !window) return KVARN_ERR_NULL;
  int st = check_cache(dst);
  if (st != KVARN_OK) return st;
  const int esz = dtype_size(dtype);
  if (!esz) return KVARN_ERR_DTYPE;
  if (!aligned16(x) || !aligned16(window)) return KVARN_ERR_ALIGN;
  if (iters < 0 || iters > 64) return KVARN_ERR_SHAPE;
  if ((int64_t)dst->batch * dst->kv_heads > INT_MAX) return KVARN_ERR_SHAPE;
  if (dst->batch == 0 || dst->kv_heads == 0 || dst->capacity == 0) return KVARN_OK;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  AppendArgs p;
  p.x = x;
  p.dtype = dtype;
  p.pos = positions;
  p.batch = dst->batch;
  p.heads = dst->kv_heads;
  p.capacity = dst->capacity;
  p.kind = dst->kind;
  p.flags = flags;
  p.codes = dst->codes;
  p.row_scale = dst->row_scale;
  p.col_scale = dst->col_scale;
  p.window = window;
  p.head_dim = cache_dim(dst);
  st = from_hip(launch_append(p, s));
  if (st != KVARN_OK) return st;
  // the chunks just filled, quantized again from the window
  QuantArgs a;
  a.x = window;
  a.dtype = dtype;
  a.head_dim = p.head_dim;
  a.sh = (int64_t)T * a.head_dim;
  a.sb = a.sh * dst->kv_heads;
  a.st = a.head_dim;
  a.batch = dst->batch;
  a.heads = dst->kv_heads;
  a.chunks = 1;
  a.chunk0 = 0;
  a.nblocks = (uint32_t)(dst->batch * dst->kv_heads);
  a.div_chunks = make_fastdiv(1u);
  a.div_heads = make_fastdiv((uint32_t)a.heads);
  a.iters = iters;
  a.flags = flags;
  a.capacity = dst->capacity;
  a.kind = dst->kind;
  a.codes = dst->codes;
  a.row_scale = dst->row_scale;
  a.col_scale = dst->col_scale;
  a.pos = positions;
  return from_hip(launch_quantize(a, s));
}

int kvarn_token_error(const void *x, int32_t dtype, int64_t stride_b, int64_t stride_h,
                      int64_t stride_t, int32_t tokens, int32_t token_offset, uint32_t flags,
                      const kvarn_cache *cache, float *ratio, float *cosine, void *stream) {
  if (flags & ~(uint32_t)KVARN_FLAG_NO_ROTATE) return KVARN_ERR_FLAGS;
  int st = check_cache(cache);
  if (st != KVARN_OK) return st;
  if (tokens < 0 || token_offset < 0) return KVARN_ERR_SHAPE;
  if (tokens == 0) return KVARN_OK;  // nothing to read or write
  if (!x || !ratio || !cosine) return KVARN_ERR_NULL;
  const int esz = dtype_size(dtype);
  if (!esz) return KVARN_ERR_DTYPE;
  if (stride_b < 0 || stride_h < 0 || stride_t < cache_dim(cache)) return KVARN_ERR_SHAPE;
  if ((int64_t)tokens + token_offset > cache->capacity) return KVARN_ERR_CAPACITY;
  if (!aligned16(x) || (stride_b * esz) % 16 || (stride_h * esz) % 16 || (stride_t * esz) % 16)
    return KVARN_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(ratio) & 3u) || (reinterpret_cast<uintptr_t>(cosine) & 3u))
    return KVARN_ERR_ALIGN;
  if ((int64_t)cache->batch * cache->kv_heads * tokens == 0) return KVARN_OK;
  DiagArgs a;
  a.x = x;
  a.dtype = dtype;
  a.sb = stride_b;
  a.sh = stride_h;
  a.st = stride_t;
  a.batch = cache->batch;
  a.heads = cache->kv_heads;
  a.tokens = tokens;
  a.token_offset = token_offset;
  a.capacity = cache->capacity;
  a.kind = cache->kind;
  a.flags = flags;
  a.codes = cache->codes;
  a.row_scale = cache->row_scale;
  a.col_scale = cache->col_scale;
  a.ratio = ratio;
  a.cosine = cosine;
  a.head_dim = cache_dim(cache);
  return from_hip(launch_token_error(a, static_cast<hipStream_t>(stream)));
}

size_t kvarn_decode_workspace_bytes_ex(int32_t batch, int32_t q_heads, int32_t capacity,
                                       int32_t head_dim) {
  if (batch < 0 || q_heads < 0 || capacity < 0 || capacity % T || !dim_ok(head_dim)) return 0;
  return decode_counter_bytes(batch, q_heads) +
         decode_partial_bytes(batch, q_heads, decode_max_wgs(capacity), head_dim);
}

size_t kvarn_decode_workspace_bytes(int32_t batch, int32_t q_heads, int32_t capacity) {
  return kvarn_decode_workspace_bytes_ex(batch, q_heads, capacity, D);
}

int kvarn_decode_attn_ex(const void *q, int32_t q_dtype, int32_t q_heads, const kvarn_cache *k,
                         const kvarn_cache *v, const int32_t *seq_lens, float softmax_scale,
                         uint32_t flags, float *out, int32_t n_split, void *workspace,
                         size_t workspace_bytes, void *stream) {
  int st = check_decode(q, q_dtype, q_heads, k, v, seq_lens, softmax_scale, flags, out, n_split);
  if (st != KVARN_OK) return st;
  if (k->batch == 0) return KVARN_OK;
  const size_t need =
      kvarn_decode_workspace_bytes_ex(k->batch, q_heads, k->capacity, cache_dim(k));
  if (!workspace) return KVARN_ERR_NULL;
  if (workspace_bytes < need) return KVARN_ERR_WORKSPACE;
  if (!aligned16(workspace)) return KVARN_ERR_ALIGN;
  // arguments are valid: from here on HIP may be queried
  const int nw = decode_wgs(q_heads, k, n_split);
  const DecodeArgs a = decode_args(q, q_dtype, q_heads, k, v, seq_lens, softmax_scale, flags,
                                   out, nw, workspace);
  return from_hip(run_decode(a, static_cast<hipStream_t>(stream)));
}

int kvarn_decode_attn_noalloc(const void *q, int32_t q_dtype, int32_t q_heads,
                              const kvarn_cache *k, const kvarn_cache *v,
                              const int32_t *seq_lens, float softmax_scale, uint32_t flags,
                              float *out, int32_t n_split, void *stream) {
  int st = check_decode(q, q_dtype, q_heads, k, v, seq_lens, softmax_scale, flags, out, n_split);
  if (st != KVARN_OK) return st;
  if (k->batch == 0) return KVARN_OK;
  const int nw = decode_wgs(q_heads, k, n_split);
  const size_t need = decode_counter_bytes(k->batch, q_heads) +
                      decode_partial_bytes(k->batch, q_heads, nw, cache_dim(k));
  if (need > (size_t)KVARN_NOALLOC_SCRATCH_BYTES) return KVARN_ERR_WORKSPACE;
  hipError_t e = hipSuccess;
  void *scratch = noalloc_scratch(&e);
  if (!scratch) return from_hip(e);
  const DecodeArgs a = decode_args(q, q_dtype, q_heads, k, v, seq_lens, softmax_scale, flags,
                                   out, nw, scratch);
  return from_hip(run_decode(a, static_cast<hipStream_t>(stream)));
}

int kvarn_decode_attn(const void *q, int32_t q_dtype, int32_t q_heads, const kvarn_cache *k,
                      const kvarn_cache *v, const int32_t *seq_lens, float softmax_scale,
                      float *out, int32_t n_split, void *workspace, size_t workspace_bytes,
                      void *stream) {
  return kvarn_decode_attn_ex(q, q_dtype, q_heads, k, v, seq_lens, softmax_scale, 0u, out,
                              n_split, workspace, workspace_bytes, stream);
}

const char *kvarn_status_string(int status) {
  switch (status) {
    case KVARN_OK: return "ok";
    case KVARN_ERR_NULL: return "null pointer argument";
    case KVARN_ERR_SHAPE: return "size, stride or count out of range";
    case KVARN_ERR_ALIGN: return "pointer or stride not 16-byte aligned";
    case KVARN_ERR_DTYPE: return "unknown dtype or cache kind";
    case KVARN_ERR_CAPACITY: return "tokens + token_offset exceed the cache capacity";
    case KVARN_ERR_WORKSPACE: return "workspace smaller than kvarn_decode_workspace_bytes";
    case KVARN_ERR_FLAGS: return "flag bit not supported by this call";
    case KVARN_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
