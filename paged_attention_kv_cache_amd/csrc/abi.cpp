// C ABI of the paged-attention library: argument validation, error
// reporting and dispatch to the HIP launchers.  Everything here runs on the
// host before any work is enqueued.  It never reads device memory, never
// allocates and never synchronises.
//
// The validation follows the error convention of the mistral.rs page
// ("Pure-Rust engines as a comparison", paged-attention section): an
// unsupported explicit setting, such as a block size outside {8, 16, 32},
// is an error, not a silent fallback.  Each message names the expected
// values and the value received.
#include <math.h>

#include <algorithm>
#include <mutex>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "pa_common.h"
#include "pa_error.h"
#include "pagedattn.h"
#include "pagedattn_kvm.h"

namespace pa {

namespace {
thread_local char g_msg[512] = "";
}

int set_error(int status, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return status;
}

int clear_error() {
  g_msg[0] = '\0';
  return PA_OK;
}

const char *last_error() { return g_msg; }

}  // namespace pa

namespace {

template <typename... A>
int fail(int status, const char *fmt, A... a) {
  return pa::set_error(status, fmt, a...);
}

int ok() { return pa::clear_error(); }

int hip_fail(hipError_t e, const char *what) {
  return fail(PA_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

int elem_bytes(int dtype) { return dtype == PA_DTYPE_BF16 ? 2 : 4; }

constexpr int kMaxGridYZ = 65535;

// value head dim of a pool (0 in the descriptor: the key head dim)
int v_dim(const pa_kv_cache *c) { return c->v_head_dim ? c->v_head_dim : c->head_dim; }

pa::CacheView view(const pa_kv_cache *c) {
  pa::CacheView v;
  v.k = c->k_cache;
  v.v = c->v_cache;
  v.num_blocks = c->num_blocks;
  v.block_size = c->block_size;
  v.num_kv_heads = c->num_kv_heads;
  v.head_dim = c->head_dim;
  v.dtype = c->dtype;
  v.head_dim_v = v_dim(c);
  return v;
}

// Cache descriptor checks shared by all entry points.  `attention` adds
// the shape limits of the attention kernels.
int check_cache(const pa_kv_cache *c, bool attention) {
  if (!c) return fail(PA_ERR_NULL, "cache descriptor is NULL");
  if (!c->k_cache || !c->v_cache)
    return fail(PA_ERR_NULL, "cache k_cache=%p v_cache=%p: both must be device pointers", c->k_cache,
                c->v_cache);
  if (c->dtype != PA_DTYPE_F32 && c->dtype != PA_DTYPE_BF16)
    return fail(PA_ERR_DTYPE, "dtype %d not in {0 (f32), 1 (bf16)}", c->dtype);
  if (c->num_blocks <= 0) return fail(PA_ERR_SHAPE, "num_blocks %d must be > 0", c->num_blocks);
  if (c->num_kv_heads <= 0) return fail(PA_ERR_SHAPE, "num_kv_heads %d must be > 0", c->num_kv_heads);
  if (c->head_dim <= 0) return fail(PA_ERR_HEAD_DIM, "head_dim %d must be > 0", c->head_dim);
  if (c->v_head_dim < 0)
    return fail(PA_ERR_HEAD_DIM, "v_head_dim %d must be > 0 (or 0: same as head_dim)", c->v_head_dim);
  if (c->block_size <= 0) return fail(PA_ERR_BLOCK_SIZE, "block_size %d must be > 0", c->block_size);
  if (attention) {
    if (c->block_size != 8 && c->block_size != 16 && c->block_size != 32)
      return fail(PA_ERR_BLOCK_SIZE, "block_size %d not in {8, 16, 32}", c->block_size);
    if (c->head_dim != 64 && c->head_dim != 128)
      return fail(PA_ERR_HEAD_DIM, "head_dim %d not in {64, 128}", c->head_dim);
    if (v_dim(c) != 64 && v_dim(c) != 128)
      return fail(PA_ERR_HEAD_DIM, "v_head_dim %d not in {64, 128}", v_dim(c));
    if (c->num_kv_heads > kMaxGridYZ)
      return fail(PA_ERR_SHAPE, "num_kv_heads %d above %d", c->num_kv_heads, kMaxGridYZ);
  }
  return PA_OK;
}

int check_heads(const pa_kv_cache *c, int num_heads) {
  if (num_heads <= 0) return fail(PA_ERR_SHAPE, "num_heads %d must be > 0", num_heads);
  if (num_heads % c->num_kv_heads)
    return fail(PA_ERR_GQA, "num_heads %d is not a multiple of num_kv_heads %d", num_heads,
                c->num_kv_heads);
  const int g = num_heads / c->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8)
    return fail(PA_ERR_GQA, "num_heads / num_kv_heads = %d not in {1, 2, 4, 8}", g);
  if (num_heads > kMaxGridYZ) return fail(PA_ERR_SHAPE, "num_heads %d above %d", num_heads, kMaxGridYZ);
  return PA_OK;
}

int num_partitions(int max_context_len, int partition_size) {
  if (partition_size <= 0 || max_context_len <= partition_size) return 1;
  return (int)(((int64_t)max_context_len + partition_size - 1) / partition_size);
}

// Workspace carve-up: m [S][H][P], l [S][H][P], o [S][H][P][D], each region
// 256-byte aligned.
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t workspace_bytes(int num_seqs, int num_heads, int head_dim, int max_context_len,
                       int partition_size) {
  if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || max_context_len <= 0 ||
      partition_size <= 0)
    return 0;
  const int P = num_partitions(max_context_len, partition_size);
  if (P <= 1) return 0;
  const size_t n = (size_t)num_seqs * num_heads * P;
  return 2 * align256(n * sizeof(float)) + align256(n * head_dim * sizeof(float));
}

int prepare_decode(const pa_kv_cache *cache, void *out, const void *q, int32_t num_seqs,
                   int32_t num_heads, const int32_t *block_tables, int32_t max_blocks_per_seq,
                   const int32_t *context_lens, int32_t max_context_len, float scale,
                   int32_t partition_size, void *workspace, size_t ws_bytes, pa::DecodeArgs *a,
                   bool split_k_workspace = true) {
  int st = check_cache(cache, true);
  if (st) return st;
  if ((st = check_heads(cache, num_heads))) return st;
  if (num_seqs < 0) return fail(PA_ERR_SHAPE, "num_seqs %d must be >= 0", num_seqs);
  if (num_seqs > kMaxGridYZ) return fail(PA_ERR_SHAPE, "num_seqs %d above %d", num_seqs, kMaxGridYZ);
  if (max_blocks_per_seq <= 0)
    return fail(PA_ERR_SHAPE, "max_blocks_per_seq %d must be > 0", max_blocks_per_seq);
  if (max_context_len < 0) return fail(PA_ERR_SHAPE, "max_context_len %d must be >= 0", max_context_len);
  if (!isfinite(scale)) return fail(PA_ERR_SHAPE, "scale %g is not finite", (double)scale);
  if (partition_size < 0 || (partition_size > 0 && partition_size % cache->block_size))
    return fail(PA_ERR_PARTITION, "partition_size %d is neither 0 nor a positive multiple of block_size %d",
                partition_size, cache->block_size);
  if (num_seqs > 0 && (!out || !q || !block_tables || !context_lens))
    return fail(PA_ERR_NULL, "out=%p q=%p block_tables=%p context_lens=%p: all must be device pointers",
                out, q, (const void *)block_tables, (const void *)context_lens);
  const int P = num_partitions(max_context_len, partition_size);
  const size_t need = split_k_workspace
                          ? workspace_bytes(num_seqs, num_heads, v_dim(cache), max_context_len, partition_size)
                          : 0;
  if (need > 0) {
    if (!workspace) return fail(PA_ERR_WORKSPACE, "workspace is NULL; %zu bytes needed", need);
    if (ws_bytes < need)
      return fail(PA_ERR_WORKSPACE, "workspace_bytes %zu < %zu needed", ws_bytes, need);
  }
  a->cache = view(cache);
  a->out = out;
  a->q = q;
  a->num_seqs = num_seqs;
  a->num_heads = num_heads;
  a->block_tables = block_tables;
  a->max_blocks_per_seq = max_blocks_per_seq;
  a->context_lens = context_lens;
  a->max_context_len = max_context_len;
  a->scale = scale;
  a->partition_size = (P > 1) ? partition_size : 0;
  a->max_partitions = P;
  a->ws_m = a->ws_l = a->ws_o = nullptr;
  if (need > 0) {
    const size_t n = (size_t)num_seqs * num_heads * P;
    char *w = static_cast<char *>(workspace);
    a->ws_m = reinterpret_cast<float *>(w);
    a->ws_l = reinterpret_cast<float *>(w + align256(n * sizeof(float)));
    a->ws_o = reinterpret_cast<float *>(w + 2 * align256(n * sizeof(float)));
  }
  return PA_OK;
}

// Split-K scratch of pa_decode_static: a file-scope device array of
// PA_STATIC_WORKSPACE_BYTES, one copy per GPU, held until the process ends.
// In host code `scratch` is only a stand-in for the symbol; its device
// address (different on every GPU) comes from hipGetSymbolAddress, once per
// device, and only that address is ever passed to a kernel.
static __device__ __align__(256) char scratch[PA_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// device address of `scratch` on the current device (looked up on the first
// call on that device); nullptr with the error recorded on failure
void *static_scratch(hipStream_t stream, int *status) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *status = hip_fail(e, "hipGetDevice");
    return nullptr;
  }
  if (stream) {
    int sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) {
      *status = hip_fail(e, "hipStreamGetDevice");
      return nullptr;
    }
    if (sdev != dev) {
      *status = fail(PA_ERR_SHAPE, "stream belongs to device %d but device %d is current", sdev, dev);
      return nullptr;
    }
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *status = fail(PA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *status = hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int pa_version(void) { return 10100; }  // 1.1.0: v_head_dim in pa_kv_cache

const char *pa_last_error_message(void) { return pa::last_error(); }

const char *pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL: return "PA_ERR_NULL";
    case PA_ERR_DTYPE: return "PA_ERR_DTYPE";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE";
    case PA_ERR_BLOCK_SIZE: return "PA_ERR_BLOCK_SIZE";
    case PA_ERR_HEAD_DIM: return "PA_ERR_HEAD_DIM";
    case PA_ERR_GQA: return "PA_ERR_GQA";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_HIP: return "PA_ERR_HIP";
    case PA_ERR_PARTITION: return "PA_ERR_PARTITION";
    case PA_ERR_NO_BLOCKS: return "PA_ERR_NO_BLOCKS";
    case PA_ERR_REQUEST: return "PA_ERR_REQUEST";
  }
  return "PA_UNKNOWN_STATUS";
}

int pa_kv_cache_write(const pa_kv_cache *cache, const void *key, const void *value,
                      const int64_t *slot_mapping, int32_t num_tokens, void *stream) {
  int st = check_cache(cache, false);
  if (st) return st;
  if (num_tokens < 0) return fail(PA_ERR_SHAPE, "num_tokens %d must be >= 0", num_tokens);
  const int64_t row_bytes = (int64_t)cache->num_kv_heads * cache->head_dim * elem_bytes(cache->dtype);
  const int64_t v_row_bytes = (int64_t)cache->num_kv_heads * v_dim(cache) * elem_bytes(cache->dtype);
  if (row_bytes % 16)
    return fail(PA_ERR_SHAPE, "num_kv_heads * head_dim * element size = %lld bytes is not a multiple of 16",
                (long long)row_bytes);
  if (v_row_bytes % 16)
    return fail(PA_ERR_SHAPE, "num_kv_heads * v_head_dim * element size = %lld bytes is not a multiple of 16",
                (long long)v_row_bytes);
  if (row_bytes > (1 << 29) || v_row_bytes > (1 << 29))
    return fail(PA_ERR_SHAPE, "rows of %lld and %lld bytes too large", (long long)row_bytes,
                (long long)v_row_bytes);
  if (num_tokens == 0) return ok();
  if (!key || !value || !slot_mapping)
    return fail(PA_ERR_NULL, "key=%p value=%p slot_mapping=%p: all must be device pointers", key, value,
                (const void *)slot_mapping);
  const int64_t num_slots = (int64_t)cache->num_blocks * cache->block_size;
  hipError_t e = pa::launch_kv_cache_write(cache->k_cache, cache->v_cache, num_slots, (int)row_bytes,
                                           (int)v_row_bytes, key, value, slot_mapping, num_tokens,
                                           (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "kv_cache_write launch");
  return ok();
}

int pa_kv_cache_copy_blocks(const pa_kv_cache *src, const pa_kv_cache *dst, const int32_t *src_ids,
                            const int32_t *dst_ids, int32_t num_copies, void *stream) {
  int st = check_cache(src, false);
  if (st) return st;
  if ((st = check_cache(dst, false))) return st;
  if (src->dtype != dst->dtype)
    return fail(PA_ERR_DTYPE, "source dtype %d differs from destination dtype %d", src->dtype, dst->dtype);
  if (src->block_size != dst->block_size || src->num_kv_heads != dst->num_kv_heads ||
      src->head_dim != dst->head_dim || v_dim(src) != v_dim(dst))
    return fail(PA_ERR_SHAPE, "block shapes differ: source (%d, %d, %d, %d), destination (%d, %d, %d, %d) as "
                "(block_size, num_kv_heads, head_dim, v_head_dim)", src->block_size, src->num_kv_heads,
                src->head_dim, v_dim(src), dst->block_size, dst->num_kv_heads, dst->head_dim, v_dim(dst));
  if (num_copies < 0) return fail(PA_ERR_SHAPE, "num_copies %d must be >= 0", num_copies);
  if ((src_ids == nullptr) != (dst_ids == nullptr))
    return fail(PA_ERR_NULL, "src_ids=%p dst_ids=%p: give both or neither", (const void *)src_ids,
                (const void *)dst_ids);
  if (!src_ids && (num_copies > src->num_blocks || num_copies > dst->num_blocks))
    return fail(PA_ERR_SHAPE, "identity copy of %d blocks: source has %d, destination %d", num_copies,
                src->num_blocks, dst->num_blocks);
  const int64_t block_bytes =
      (int64_t)src->block_size * src->num_kv_heads * src->head_dim * elem_bytes(src->dtype);
  const int64_t v_block_bytes =
      (int64_t)src->block_size * src->num_kv_heads * v_dim(src) * elem_bytes(src->dtype);
  if (block_bytes % 16 || v_block_bytes % 16)
    return fail(PA_ERR_SHAPE, "a block is %lld bytes of K and %lld of V, not multiples of 16",
                (long long)block_bytes, (long long)v_block_bytes);
  if (num_copies == 0) return ok();
  hipError_t e = pa::launch_kv_cache_copy_blocks(src->k_cache, src->v_cache, dst->k_cache, dst->v_cache,
                                                 src->num_blocks, dst->num_blocks, block_bytes, v_block_bytes,
                                                 src_ids, dst_ids, num_copies, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "kv_cache_copy_blocks launch");
  return ok();
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_size) {
  return workspace_bytes(num_seqs, num_heads, head_dim, max_context_len, partition_size);
}

int pa_decode_partition(const pa_kv_cache *cache, void *out, const void *q, int32_t num_seqs,
                        int32_t num_heads, const int32_t *block_tables, int32_t max_blocks_per_seq,
                        const int32_t *context_lens, int32_t max_context_len, float scale,
                        int32_t partition_size, void *workspace, size_t workspace_bytes,
                        void *stream) {
  pa::DecodeArgs a;
  int st = prepare_decode(cache, out, q, num_seqs, num_heads, block_tables, max_blocks_per_seq,
                          context_lens, max_context_len, scale, partition_size, workspace,
                          workspace_bytes, &a);
  if (st) return st;
  if (num_seqs == 0) return ok();
  hipError_t e = pa::launch_decode_partition(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "decode partition launch");
  return ok();
}

int pa_decode_reduce(void *out, int32_t dtype, int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                     const int32_t *context_lens, int32_t max_context_len, int32_t partition_size,
                     const void *workspace, size_t ws_bytes, void *stream) {
  if (dtype != PA_DTYPE_F32 && dtype != PA_DTYPE_BF16)
    return fail(PA_ERR_DTYPE, "dtype %d not in {0 (f32), 1 (bf16)}", dtype);
  if (head_dim != 64 && head_dim != 128) return fail(PA_ERR_HEAD_DIM, "head_dim %d not in {64, 128}", head_dim);
  if (num_seqs < 0 || num_seqs > kMaxGridYZ)
    return fail(PA_ERR_SHAPE, "num_seqs %d not in [0, %d]", num_seqs, kMaxGridYZ);
  if (num_heads <= 0 || num_heads > kMaxGridYZ)
    return fail(PA_ERR_SHAPE, "num_heads %d not in [1, %d]", num_heads, kMaxGridYZ);
  if (max_context_len < 0) return fail(PA_ERR_SHAPE, "max_context_len %d must be >= 0", max_context_len);
  if (partition_size < 0) return fail(PA_ERR_PARTITION, "partition_size %d must be >= 0", partition_size);
  const int P = num_partitions(max_context_len, partition_size);
  if (num_seqs == 0 || P <= 1) return ok();
  if (!out || !context_lens)
    return fail(PA_ERR_NULL, "out=%p context_lens=%p: both must be device pointers", out,
                (const void *)context_lens);
  const size_t need = workspace_bytes(num_seqs, num_heads, head_dim, max_context_len, partition_size);
  if (!workspace) return fail(PA_ERR_WORKSPACE, "workspace is NULL; %zu bytes needed", need);
  if (ws_bytes < need) return fail(PA_ERR_WORKSPACE, "workspace_bytes %zu < %zu needed", ws_bytes, need);
  pa::DecodeArgs a{};
  a.cache.dtype = dtype;
  a.cache.head_dim = head_dim;
  a.cache.head_dim_v = head_dim;  // the output row width
  a.cache.block_size = 1;  // unused by the reduce
  a.cache.num_kv_heads = 1;
  a.out = out;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.context_lens = context_lens;
  a.max_context_len = max_context_len;
  a.max_blocks_per_seq = max_context_len;  // with block_size 1: no extra cap
  a.partition_size = partition_size;
  a.max_partitions = P;
  const size_t n = (size_t)num_seqs * num_heads * P;
  char *w = static_cast<char *>(const_cast<void *>(workspace));
  a.ws_m = reinterpret_cast<float *>(w);
  a.ws_l = reinterpret_cast<float *>(w + align256(n * sizeof(float)));
  a.ws_o = reinterpret_cast<float *>(w + 2 * align256(n * sizeof(float)));
  hipError_t e = pa::launch_decode_reduce(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "decode reduce launch");
  return ok();
}

int pa_decode(const pa_kv_cache *cache, void *out, const void *q, int32_t num_seqs, int32_t num_heads,
              const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
              int32_t max_context_len, float scale, int32_t partition_size, void *workspace,
              size_t workspace_bytes, void *stream) {
  pa::DecodeArgs a;
  int st = prepare_decode(cache, out, q, num_seqs, num_heads, block_tables, max_blocks_per_seq,
                          context_lens, max_context_len, scale, partition_size, workspace,
                          workspace_bytes, &a);
  if (st) return st;
  if (num_seqs == 0) return ok();
  hipError_t e = pa::launch_decode_partition(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "decode partition launch");
  e = pa::launch_decode_reduce(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "decode reduce launch");
  return ok();
}

int pa_decode_static(const pa_kv_cache *cache, void *out, const void *q, int32_t num_seqs, int32_t num_heads,
                     const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
                     int32_t max_context_len, float scale, int32_t partition_size, void *stream) {
  // the split-K size check comes before any HIP call, so an oversized
  // request is refused without touching the device
  int st = check_cache(cache, true);
  if (st) return st;
  const size_t need = workspace_bytes(num_seqs, num_heads, v_dim(cache), max_context_len, partition_size);
  if (need > (size_t)PA_STATIC_WORKSPACE_BYTES)
    return fail(PA_ERR_WORKSPACE,
                "split-K partials need %zu bytes, above the static scratch of %zu bytes; use a larger "
                "partition_size or pa_decode with a caller workspace",
                need, (size_t)PA_STATIC_WORKSPACE_BYTES);
  void *ws = nullptr;
  if (need > 0) {
    // validate the rest before the first device query
    pa::DecodeArgs probe;
    st = prepare_decode(cache, out, q, num_seqs, num_heads, block_tables, max_blocks_per_seq, context_lens,
                        max_context_len, scale, partition_size, nullptr, 0, &probe, false);
    if (st) return st;
    if (num_seqs == 0) return ok();
    ws = static_scratch((hipStream_t)stream, &st);
    if (!ws) return st;
  }
  return pa_decode(cache, out, q, num_seqs, num_heads, block_tables, max_blocks_per_seq, context_lens,
                   max_context_len, scale, partition_size, ws, need, stream);
}

int pa_decode_append(const pa_kv_cache *cache, void *out, const void *q, const void *key, const void *value,
                     int32_t num_seqs, int32_t num_heads, const int32_t *block_tables, int32_t max_blocks_per_seq,
                     const int32_t *context_lens, int32_t max_context_len, float scale, int32_t partition_size,
                     void *workspace, size_t workspace_bytes, void *stream) {
  pa::DecodeArgs a;
  int st = prepare_decode(cache, out, q, num_seqs, num_heads, block_tables, max_blocks_per_seq, context_lens,
                          max_context_len, scale, partition_size, workspace, workspace_bytes, &a);
  if (st) return st;
  const int64_t k_row = (int64_t)cache->num_kv_heads * cache->head_dim * elem_bytes(cache->dtype);
  const int64_t v_row = (int64_t)cache->num_kv_heads * v_dim(cache) * elem_bytes(cache->dtype);
  if (k_row % 16 || v_row % 16)
    return fail(PA_ERR_SHAPE, "K and V rows of %lld and %lld bytes are not multiples of 16", (long long)k_row,
                (long long)v_row);
  if (num_seqs == 0) return ok();
  if (!key || !value)
    return fail(PA_ERR_NULL, "key=%p value=%p: both must be device pointers", key, value);
  a.new_k = key;
  a.new_v = value;
  hipError_t e;
  if (!pa::decode_fast_path(a)) {
    // shapes the matrix-core kernel does not take (fp32 pools): the cache
    // write first, then the plain decode, which reads the new rows from the
    // cache
    e = pa::launch_kv_cache_append(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "decode append write launch");
    a.new_k = a.new_v = nullptr;
  }
  e = pa::launch_decode_partition(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "decode partition launch");
  e = pa::launch_decode_reduce(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "decode reduce launch");
  return ok();
}

// cascade decode: tokens per chunk of the shared part (one partial slot
// each, and one work-group per 16 of its columns).  Longer chunks mean
// fewer slots for the reduce to merge; 512 was the fastest of 128, 256 and
// 512 on the prefix-shared batches.
constexpr int kCascadeChunk = 512;

// slots per (row, head): chunks of the shared part, then partitions of the
// row's own tokens
int cascade_slots(int max_context_len, int partition_size) {
  const int c = std::max(1, (max_context_len + kCascadeChunk - 1) / kCascadeChunk);
  return c + std::max(1, num_partitions(max_context_len, partition_size));
}

size_t pa_decode_cascade_workspace_bytes(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                         int32_t max_context_len, int32_t partition_size) {
  if (num_seqs <= 0 || num_heads <= 0 || head_dim <= 0 || max_context_len < 0 || partition_size <= 0) return 0;
  const size_t P = (size_t)cascade_slots(max_context_len, partition_size);
  const size_t n = (size_t)num_seqs * num_heads * P;
  return 2 * align256(n * sizeof(float)) + align256(n * head_dim * sizeof(float));
}

int pa_decode_cascade(const pa_kv_cache *cache, void *out, const void *q, int32_t num_seqs, int32_t num_heads,
                      const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
                      int32_t max_context_len, float scale, int32_t partition_size, int32_t num_groups,
                      const int32_t *group_start, const int32_t *shared_len, int32_t max_group_size,
                      int32_t max_shared_len, void *workspace, size_t workspace_bytes, void *stream) {
  if (partition_size <= 0)
    return fail(PA_ERR_PARTITION, "cascade decode needs partition_size > 0 (a multiple of block_size), got %d",
                partition_size);
  pa::DecodeArgs a;
  // validation of the shared arguments (the plain-decode workspace check is
  // replaced by the cascade one below)
  int st = prepare_decode(cache, out, q, num_seqs, num_heads, block_tables, max_blocks_per_seq, context_lens,
                          max_context_len, scale, partition_size, nullptr, 0, &a, false);
  if (st) return st;
  if (cache->dtype != PA_DTYPE_BF16)
    return fail(PA_ERR_UNSUPPORTED, "cascade decode is bf16 only (dtype %d)", cache->dtype);
  if (num_groups < 0 || (num_seqs > 0 && num_groups == 0))
    return fail(PA_ERR_SHAPE, "num_groups %d: every sequence belongs to one group", num_groups);
  if (num_groups > kMaxGridYZ) return fail(PA_ERR_SHAPE, "num_groups %d above %d", num_groups, kMaxGridYZ);
  if (num_seqs == 0) return ok();
  if (!group_start || !shared_len)
    return fail(PA_ERR_NULL, "group_start=%p shared_len=%p: both must be device pointers",
                (const void *)group_start, (const void *)shared_len);
  if (max_group_size <= 0 || max_group_size > num_seqs)
    return fail(PA_ERR_SHAPE, "max_group_size %d not in [1, num_seqs %d]", max_group_size, num_seqs);
  if (max_shared_len < 0) return fail(PA_ERR_SHAPE, "max_shared_len %d must be >= 0", max_shared_len);
  const int P = cascade_slots(max_context_len, partition_size);
  const size_t need = pa_decode_cascade_workspace_bytes(num_seqs, num_heads, v_dim(cache), max_context_len,
                                                        partition_size);
  if (!workspace) return fail(PA_ERR_WORKSPACE, "workspace is NULL; %zu bytes needed", need);
  if (workspace_bytes < need) return fail(PA_ERR_WORKSPACE, "workspace_bytes %zu < %zu needed", workspace_bytes, need);
  const size_t n = (size_t)num_seqs * num_heads * P;
  char *w = static_cast<char *>(workspace);
  a.ws_m = reinterpret_cast<float *>(w);
  a.ws_l = reinterpret_cast<float *>(w + align256(n * sizeof(float)));
  a.ws_o = reinterpret_cast<float *>(w + 2 * align256(n * sizeof(float)));
  a.partition_size = partition_size;
  a.max_partitions = P;
  a.group_start = group_start;
  a.shared_len = shared_len;
  a.num_groups = num_groups;
  const int chunk = kCascadeChunk;
  a.shared_chunk = chunk;

  // chunks per group: enough for max_shared_len.  shared_len is clamped to
  // the tokens those chunks cover (a multiple of 512, so of block_size);
  // the members' partitions read anything past it.
  a.shared_chunks = std::max(1, (std::min(max_shared_len, max_context_len) + chunk - 1) / chunk);
  a.shared_cap = a.shared_chunks * chunk;
  a.max_group_size = max_group_size;
  const int col_tiles = (max_group_size * (num_heads / cache->num_kv_heads) + 15) / 16;
  const int grid_z = pa::cascade_grid_z(a, col_tiles);
  if (grid_z > kMaxGridYZ || (int64_t)grid_z * num_seqs > INT32_MAX)
    return fail(PA_ERR_SHAPE,
                "cascade launch needs %d grid rows of %d items (shared chunks x column tiles per group, then own "
                "partitions), above %d; lower max_shared_len or max_group_size, or raise partition_size",
                grid_z, num_seqs, kMaxGridYZ);
  // 1-2. every group's shared chunks, once for all its rows, and every
  // row's own tokens after them, in one launch
  hipError_t e = pa::launch_decode_partition(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "cascade partition launch");
  // 3. merge all slots
  e = pa::launch_decode_reduce(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "cascade reduce launch");
  return ok();
}

int pa_prefill_chunk(const pa_kv_cache *cache, void *out, const void *q, const int32_t *query_start_loc,
                     int32_t num_seqs, int32_t num_heads, int32_t num_query_tokens, int32_t max_query_len,
                     const int32_t *block_tables, int32_t max_blocks_per_seq, const int32_t *context_lens,
                     int32_t max_context_len, float scale, void *stream) {
  int st = check_cache(cache, true);
  if (st) return st;
  if ((st = check_heads(cache, num_heads))) return st;
  if (num_seqs < 0 || num_seqs > kMaxGridYZ)
    return fail(PA_ERR_SHAPE, "num_seqs %d not in [0, %d]", num_seqs, kMaxGridYZ);
  if (num_query_tokens < 0) return fail(PA_ERR_SHAPE, "num_query_tokens %d must be >= 0", num_query_tokens);
  if (max_query_len < 0) return fail(PA_ERR_SHAPE, "max_query_len %d must be >= 0", max_query_len);
  if (max_blocks_per_seq <= 0)
    return fail(PA_ERR_SHAPE, "max_blocks_per_seq %d must be > 0", max_blocks_per_seq);
  if (max_context_len < 0) return fail(PA_ERR_SHAPE, "max_context_len %d must be >= 0", max_context_len);
  if (!isfinite(scale)) return fail(PA_ERR_SHAPE, "scale %g is not finite", (double)scale);
  if (num_seqs == 0 || num_query_tokens == 0 || max_query_len == 0) return ok();
  if (!out || !q || !query_start_loc || !block_tables || !context_lens)
    return fail(PA_ERR_NULL,
                "out=%p q=%p query_start_loc=%p block_tables=%p context_lens=%p: all must be device pointers",
                out, q, (const void *)query_start_loc, (const void *)block_tables, (const void *)context_lens);
  if (cache->dtype == PA_DTYPE_F32) {
    // fp32: one single-pass row of the generic decode kernel per packed
    // query row, over its sequence's keys up to the row's own position
    if (num_query_tokens > kMaxGridYZ)
      return fail(PA_ERR_UNSUPPORTED, "fp32 prefill_chunk takes at most %d query rows, got %d", kMaxGridYZ,
                  num_query_tokens);
    pa::DecodeArgs d;
    d.cache = view(cache);
    d.out = out;
    d.q = q;
    d.num_seqs = num_query_tokens;
    d.num_heads = num_heads;
    d.block_tables = block_tables;
    d.max_blocks_per_seq = max_blocks_per_seq;
    d.context_lens = context_lens;
    d.max_context_len = max_context_len;
    d.scale = scale;
    d.partition_size = 0;
    d.max_partitions = 1;
    d.ws_m = d.ws_l = d.ws_o = nullptr;
    d.query_start_loc = query_start_loc;
    d.num_prefill_seqs = num_seqs;
    hipError_t e = pa::launch_decode_partition(d, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "fp32 prefill_chunk launch");
    return ok();
  }
  pa::PrefillArgs a;
  a.cache = view(cache);
  a.out = out;
  a.q = q;
  a.query_start_loc = query_start_loc;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_query_tokens = num_query_tokens;
  a.max_query_len = max_query_len;
  a.block_tables = block_tables;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.context_lens = context_lens;
  a.max_context_len = max_context_len;
  a.scale = scale;
  hipError_t e = pa::launch_prefill_chunk(a, (hipStream_t)stream);
  if (e == hipErrorNotSupported)
    return fail(PA_ERR_UNSUPPORTED,
                "prefill_chunk: head_dim %d, v_head_dim %d with num_heads/num_kv_heads %d not built",
                cache->head_dim, v_dim(cache), num_heads / cache->num_kv_heads);
  if (e != hipSuccess) return hip_fail(e, "prefill_chunk launch");
  return ok();
}

}  // extern "C"
