// Native serving step (include/pagedattn_serve.h): the step scheduler
// plans into pinned host memory, one asynchronous copy moves the step's
// arrays to the device, and the step's K/V write and attention are
// launched from here.  The alternating prompt / decode schedule and the
// 4096-token budget with 512-token chunks are those of the scheduling
// section of the mistral.rs comparison page (in pagedattn_kvm.h); the
// write-then-attend order of a step is that of the TensorSharp Mistral 3
// page, section 3.
#include <hip/hip_runtime.h>

#include <cstring>
#include <new>

#include "pa_error.h"
#include "pagedattn.h"
#include "pagedattn_kvm.h"
#include "pagedattn_serve.h"

namespace {

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// byte offsets of a step's arrays in the device buffer (and in the front of
// each staging buffer, which is copied as one block), then the request ids,
// which only the host reads
struct Layout {
  size_t slots, qsl, ctx, tab, meta, ids, staging;
};

bool layout(int32_t cap_seqs, int32_t cap_blocks, int32_t cap_tokens, Layout &L) {
  if (cap_seqs <= 0 || cap_blocks <= 0 || cap_tokens <= 0) return false;
  L.slots = 0;
  L.qsl = L.slots + sizeof(int64_t) * (size_t)cap_tokens;
  L.ctx = L.qsl + sizeof(int32_t) * ((size_t)cap_seqs + 1);
  L.tab = L.ctx + sizeof(int32_t) * (size_t)cap_seqs;
  L.meta = align_up(L.tab + sizeof(int32_t) * (size_t)cap_seqs * (size_t)cap_blocks, 256);
  L.ids = L.meta;
  L.staging = L.ids + sizeof(int64_t) * (size_t)cap_seqs;
  return true;
}

}  // namespace

struct pa_serve {
  pa_sched *sched = nullptr;
  int32_t num_heads = 0, partition_size = 0, mixed_split_context = 0;
  float scale = 0.f;
  int32_t cap_seqs = 0, cap_blocks = 0, cap_tokens = 0;
  Layout L{};
  char *dev_meta = nullptr;
  char *staging[2] = {nullptr, nullptr};
  hipEvent_t copied[2] = {nullptr, nullptr};
  bool in_flight[2] = {false, false};  // a copy out of this buffer was enqueued
  int next = 0;                        // staging buffer of the next plan
  bool planned = false;                // a plan waits for attend / complete
  pa_step step{};
};

extern "C" size_t pa_serve_meta_bytes(int32_t max_seqs, int32_t max_blocks_per_seq, int32_t max_tokens) {
  Layout L;
  return layout(max_seqs, max_blocks_per_seq, max_tokens, L) ? L.meta : 0;
}

extern "C" void pa_serve_destroy(pa_serve *s) {
  if (!s) return;
  for (int i = 0; i < 2; ++i) {
    if (s->copied[i]) {
      if (s->in_flight[i]) (void)hipEventSynchronize(s->copied[i]);
      (void)hipEventDestroy(s->copied[i]);
    }
    if (s->staging[i]) (void)hipHostFree(s->staging[i]);
  }
  delete s;
}

extern "C" pa_serve *pa_serve_create(pa_sched *sched, int32_t num_heads, float scale, int32_t partition_size,
                                     int32_t mixed_split_context, int32_t max_seqs, int32_t max_blocks_per_seq,
                                     int32_t max_tokens, void *dev_meta, size_t dev_meta_bytes) {
  Layout L;
  if (!sched || !dev_meta) {
    pa::set_error(PA_ERR_NULL, "sched=%p dev_meta=%p: both are required", (void *)sched, dev_meta);
    return nullptr;
  }
  if (!layout(max_seqs, max_blocks_per_seq, max_tokens, L) || num_heads <= 0) {
    pa::set_error(PA_ERR_SHAPE, "capacities %d seqs, %d blocks, %d tokens and %d heads must be positive", max_seqs,
                  max_blocks_per_seq, max_tokens, num_heads);
    return nullptr;
  }
  if (dev_meta_bytes < L.meta) {
    pa::set_error(PA_ERR_SHAPE, "dev_meta holds %zu bytes, the step arrays need %zu", dev_meta_bytes, L.meta);
    return nullptr;
  }
  if (partition_size < 0) {
    pa::set_error(PA_ERR_PARTITION, "partition_size %d must be >= 0", partition_size);
    return nullptr;
  }
  if (mixed_split_context < 0) {
    pa::set_error(PA_ERR_SHAPE, "mixed_split_context %d must be >= 0", mixed_split_context);
    return nullptr;
  }
  pa_serve *s = new (std::nothrow) pa_serve();
  if (!s) {
    pa::set_error(PA_ERR_SHAPE, "out of host memory");
    return nullptr;
  }
  s->sched = sched;
  s->num_heads = num_heads;
  s->scale = scale;
  s->partition_size = partition_size;
  s->mixed_split_context = mixed_split_context;
  s->cap_seqs = max_seqs;
  s->cap_blocks = max_blocks_per_seq;
  s->cap_tokens = max_tokens;
  s->L = L;
  s->dev_meta = static_cast<char *>(dev_meta);
  for (int i = 0; i < 2; ++i) {
    hipError_t e = hipHostMalloc((void **)&s->staging[i], L.staging, hipHostMallocDefault);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&s->copied[i], hipEventDisableTiming);
    if (e != hipSuccess) {
      pa::set_error(PA_ERR_HIP, "pinned staging or event: HIP error %d (%s)", (int)e, hipGetErrorString(e));
      pa_serve_destroy(s);
      return nullptr;
    }
    std::memset(s->staging[i], 0, L.staging);
  }
  pa::clear_error();
  return s;
}

extern "C" int pa_serve_plan(pa_serve *s, pa_step *out, void *stream) {
  if (!s || !out) return pa::set_error(PA_ERR_NULL, "serve object or step is NULL");
  if (s->planned) return pa::set_error(PA_ERR_SHAPE, "the previous step was planned but not completed");
  const int b = s->next;
  if (s->in_flight[b]) {
    // the copy out of this buffer (two plans ago) must have run
    const hipError_t e = hipEventSynchronize(s->copied[b]);
    if (e != hipSuccess) return pa::set_error(PA_ERR_HIP, "staging event: HIP error %d (%s)", (int)e, hipGetErrorString(e));
    s->in_flight[b] = false;
  }
  char *buf = s->staging[b];
  pa_step &st = s->step;
  std::memset(&st, 0, sizeof(st));
  st.request_ids = reinterpret_cast<int64_t *>(buf + s->L.ids);
  st.slot_mapping = reinterpret_cast<int64_t *>(buf + s->L.slots);
  st.query_start_loc = reinterpret_cast<int32_t *>(buf + s->L.qsl);
  st.context_lens = reinterpret_cast<int32_t *>(buf + s->L.ctx);
  st.block_tables = reinterpret_cast<int32_t *>(buf + s->L.tab);
  st.cap_seqs = s->cap_seqs;
  st.cap_tokens = s->cap_tokens;
  st.cap_blocks = s->cap_blocks;
  const int rc = pa_sched_next_step(s->sched, &st);
  *out = st;
  if (rc) return rc;
  if (st.kind == 0) return pa::clear_error();
  const hipError_t e = hipMemcpyAsync(s->dev_meta, buf, s->L.meta, hipMemcpyHostToDevice, (hipStream_t)stream);
  if (e != hipSuccess) return pa::set_error(PA_ERR_HIP, "step copy: HIP error %d (%s)", (int)e, hipGetErrorString(e));
  const hipError_t r = hipEventRecord(s->copied[b], (hipStream_t)stream);
  if (r != hipSuccess) return pa::set_error(PA_ERR_HIP, "staging event: HIP error %d (%s)", (int)r, hipGetErrorString(r));
  s->in_flight[b] = true;
  s->next = 1 - b;
  s->planned = true;
  return pa::clear_error();
}

extern "C" int pa_serve_attend(pa_serve *s, const pa_kv_cache *cache, const void *new_key, const void *new_value,
                               const void *q, void *out, void *workspace, size_t workspace_bytes, void *stream) {
  if (!s) return pa::set_error(PA_ERR_NULL, "serve object is NULL");
  if (!s->planned) return pa::set_error(PA_ERR_SHAPE, "no step is planned");
  const pa_step &st = s->step;
  const int64_t *d_slots = reinterpret_cast<const int64_t *>(s->dev_meta + s->L.slots);
  const int32_t *d_qsl = reinterpret_cast<const int32_t *>(s->dev_meta + s->L.qsl);
  const int32_t *d_ctx = reinterpret_cast<const int32_t *>(s->dev_meta + s->L.ctx);
  const int32_t *d_tab = reinterpret_cast<const int32_t *>(s->dev_meta + s->L.tab);
  int rc = pa_kv_cache_write(cache, new_key, new_value, d_slots, st.num_tokens, stream);
  if (rc) return rc;
  int nd = 0;  // leading one-token rows (a mixed step's decode rows)
  int32_t longest = 0, longest_chunk = 0;
  if (st.kind == 3 && s->partition_size > 0 && s->mixed_split_context > 0) {
    for (; nd < st.num_seqs && st.query_start_loc[nd + 1] - st.query_start_loc[nd] == 1; ++nd)
      longest = st.context_lens[nd] > longest ? st.context_lens[nd] : longest;
    for (int i = nd; i < st.num_seqs; ++i)
      longest_chunk = st.context_lens[i] > longest_chunk ? st.context_lens[i] : longest_chunk;
  }
  // the decode rows are worth a launch of their own when one of them is long
  // and longer than every chunk's context (else a chunk's items, which read
  // as many keys, set the prefill launch's time anyway)
  if (nd > 0 && longest >= s->mixed_split_context && longest > longest_chunk) {
    // A mixed step's decode rows through split-K decode (a long context
    // spread over many work-groups instead of one per kv head), the prompt
    // chunks after them through the prefill kernel.  A one-token row is a
    // decode step under the causal alignment; packed row i is decode row i,
    // and the chunks' query offsets are absolute rows of the same q and out.
    rc = pa_decode(cache, out, q, nd, s->num_heads, d_tab, st.cap_blocks, d_ctx, st.max_context_len, s->scale,
                   s->partition_size, workspace, workspace_bytes, stream);
    if (rc || nd == st.num_seqs) return rc;
    return pa_prefill_chunk(cache, out, q, d_qsl + nd, st.num_seqs - nd, s->num_heads, st.num_tokens,
                            st.max_query_len, d_tab + (size_t)nd * st.cap_blocks, st.cap_blocks, d_ctx + nd,
                            st.max_context_len, s->scale, stream);
  }
  if (st.kind == 1 || st.kind == 3)
    return pa_prefill_chunk(cache, out, q, d_qsl, st.num_seqs, s->num_heads, st.num_tokens, st.max_query_len, d_tab,
                            st.cap_blocks, d_ctx, st.max_context_len, s->scale, stream);
  return pa_decode(cache, out, q, st.num_seqs, s->num_heads, d_tab, st.cap_blocks, d_ctx, st.max_context_len,
                   s->scale, s->partition_size, workspace, workspace_bytes, stream);
}

extern "C" int pa_serve_complete(pa_serve *s, const int32_t *sampled, int32_t *num_finished) {
  if (!s || !num_finished) return pa::set_error(PA_ERR_NULL, "serve object or num_finished is NULL");
  if (!s->planned) return pa::set_error(PA_ERR_SHAPE, "no step is planned");
  const int rc = pa_sched_complete_step(s->sched, &s->step, sampled, num_finished);
  if (rc) return rc;
  s->planned = false;
  return pa::clear_error();
}
