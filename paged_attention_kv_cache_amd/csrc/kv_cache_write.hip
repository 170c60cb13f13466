// Slot-mapping scatter of new tokens' K and V into the paged KV pool.
//
// TensorSharp, Mistral 3 page, section 11 "Batched / paged forward": fresh
// K and V are written into the layer's paged buffer at
// blockId * blockSize + offset, with no per-sequence extract/inject.  The
// buffer's flat order [numBlocks, blockSize, numKvHeads, headDim] makes one
// slot's K (or V) for all kv heads one contiguous row of
// num_kv_heads * head_dim elements, so the scatter is a row copy.  K and V
// rows may differ in width (separate key and value head dims, section 4.1).
//
// One thread moves one 16-byte chunk with a 128-bit load and store: the
// threads of a token cover its K row's chunks, then its V row's, so each
// row is read and written fully coalesced.  The copy moves bits and does
// no arithmetic, so it is exact for any element type.
#include "pa_common.h"

namespace pa {

__global__ void __launch_bounds__(256)
kv_cache_write_kernel(uint4 *__restrict__ k_cache, uint4 *__restrict__ v_cache, int64_t num_slots,
                      int k_chunks, int v_chunks, const uint4 *__restrict__ key,
                      const uint4 *__restrict__ value, const int64_t *__restrict__ slots,
                      int num_tokens) {
  const int per_token = k_chunks + v_chunks;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t token = gid / per_token;
  int chunk = (int)(gid - token * per_token);
  if (token >= num_tokens) return;
  const int64_t slot = slots[token];
  if (slot < 0 || slot >= num_slots) return;  // padding, or outside the pool
  if (chunk < k_chunks) {
    k_cache[slot * k_chunks + chunk] = key[token * k_chunks + chunk];
  } else {
    chunk -= k_chunks;
    v_cache[slot * v_chunks + chunk] = value[token * v_chunks + chunk];
  }
}

hipError_t launch_kv_cache_write(void *k_cache, void *v_cache, int64_t num_slots, int k_row_bytes,
                                 int v_row_bytes, const void *key, const void *value, const int64_t *slots,
                                 int num_tokens, hipStream_t stream) {
  const int k_chunks = k_row_bytes / 16, v_chunks = v_row_bytes / 16;
  const int64_t total = (int64_t)num_tokens * (k_chunks + v_chunks);
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(kv_cache_write_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     static_cast<uint4 *>(k_cache), static_cast<uint4 *>(v_cache), num_slots, k_chunks,
                     v_chunks, static_cast<const uint4 *>(key), static_cast<const uint4 *>(value), slots,
                     num_tokens);
  return hipGetLastError();
}

// Whole-block copy between pools of the same block shape (or inside one
// pool): growing a pool into a larger allocation keeps the K/V of the
// sequences already placed (TensorSharp, Mistral 3 page, section 11, the
// grow path of the paged buffers), and a block-id map copies shared blocks
// for a sequence that must write into its own copy.  A block of K is
// block_size * num_kv_heads * head_dim contiguous elements (of V, the same
// with the value head dim); the grid walks 16-byte chunks of every
// (copy, K then V) with 128-bit loads and stores.  Copies whose ids fall
// outside either pool are skipped.
__global__ void __launch_bounds__(256)
kv_cache_copy_blocks_kernel(const uint4 *__restrict__ src_k, const uint4 *__restrict__ src_v,
                            uint4 *__restrict__ dst_k, uint4 *__restrict__ dst_v, int src_blocks,
                            int dst_blocks, int64_t k_chunks, int64_t v_chunks,
                            const int32_t *__restrict__ src_ids, const int32_t *__restrict__ dst_ids,
                            int num_copies) {
  const int64_t per_copy = k_chunks + v_chunks;  // K then V
  const int64_t total = (int64_t)num_copies * per_copy;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
       g += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = g / per_copy;
    int64_t r = g - c * per_copy;
    const bool is_v = r >= k_chunks;
    if (is_v) r -= k_chunks;
    const int64_t chunks = is_v ? v_chunks : k_chunks;
    const int sb = src_ids ? src_ids[c] : (int)c;
    const int db = dst_ids ? dst_ids[c] : (int)c;
    if ((unsigned)sb >= (unsigned)src_blocks || (unsigned)db >= (unsigned)dst_blocks) continue;
    const uint4 x = (is_v ? src_v : src_k)[(int64_t)sb * chunks + r];
    (is_v ? dst_v : dst_k)[(int64_t)db * chunks + r] = x;
  }
}

hipError_t launch_kv_cache_copy_blocks(const void *src_k, const void *src_v, void *dst_k, void *dst_v,
                                       int src_blocks, int dst_blocks, int64_t k_block_bytes,
                                       int64_t v_block_bytes, const int32_t *src_ids, const int32_t *dst_ids,
                                       int num_copies, hipStream_t stream) {
  const int64_t kc = k_block_bytes / 16, vc = v_block_bytes / 16;
  const int64_t total = (int64_t)num_copies * (kc + vc);
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;  // grid-stride beyond this
  hipLaunchKernelGGL(kv_cache_copy_blocks_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     static_cast<const uint4 *>(src_k), static_cast<const uint4 *>(src_v),
                     static_cast<uint4 *>(dst_k), static_cast<uint4 *>(dst_v), src_blocks, dst_blocks, kc, vc,
                     src_ids, dst_ids, num_copies);
  return hipGetLastError();
}

// Cache write of a fused append on the shapes the fast decode kernel does
// not take: sequence i's new K and V rows go to the slot of its position
// context_len - 1, found through its block table (the slot mapping a decode
// step would pass to the scatter above).  One thread per 16-byte chunk, K
// chunks then V chunks of each sequence.
__global__ void __launch_bounds__(256)
kv_cache_append_kernel(uint4 *__restrict__ k_cache, uint4 *__restrict__ v_cache, int num_blocks, int block_shift,
                       int k_chunks, int v_chunks, const uint4 *__restrict__ key, const uint4 *__restrict__ value,
                       const int32_t *__restrict__ block_tables, int max_blocks_per_seq,
                       const int32_t *__restrict__ context_lens, int ctx_cap, int num_seqs) {
  const int per_seq = k_chunks + v_chunks;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t seq = gid / per_seq;
  int chunk = (int)(gid - seq * per_seq);
  if (seq >= num_seqs) return;
  int ctx = context_lens[seq];
  ctx = ctx < ctx_cap ? ctx : ctx_cap;
  if (ctx <= 0) return;
  const int pos = ctx - 1;
  const int blk = block_tables[seq * (int64_t)max_blocks_per_seq + (pos >> block_shift)];
  if ((unsigned)blk >= (unsigned)num_blocks) return;
  const int64_t slot = ((int64_t)blk << block_shift) + (pos & ((1 << block_shift) - 1));
  if (chunk < k_chunks) {
    k_cache[slot * k_chunks + chunk] = key[seq * k_chunks + chunk];
  } else {
    chunk -= k_chunks;
    v_cache[slot * v_chunks + chunk] = value[seq * v_chunks + chunk];
  }
}

hipError_t launch_kv_cache_append(const DecodeArgs &a, hipStream_t stream) {
  const int eb = a.cache.dtype == 1 ? 2 : 4;
  const int k_chunks = a.cache.num_kv_heads * a.cache.head_dim * eb / 16;
  const int v_chunks = a.cache.num_kv_heads * a.cache.head_dim_v * eb / 16;
  const int64_t total = (int64_t)a.num_seqs * (k_chunks + v_chunks);
  if (total == 0) return hipSuccess;
  int shift = 0;
  while ((1 << shift) < a.cache.block_size) ++shift;
  const int64_t table_cap = (int64_t)a.max_blocks_per_seq * a.cache.block_size;
  const int ctx_cap = (int)(table_cap < a.max_context_len ? table_cap : a.max_context_len);
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(kv_cache_append_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     static_cast<uint4 *>(const_cast<void *>(a.cache.k)),
                     static_cast<uint4 *>(const_cast<void *>(a.cache.v)), a.cache.num_blocks, shift, k_chunks,
                     v_chunks, static_cast<const uint4 *>(a.new_k), static_cast<const uint4 *>(a.new_v),
                     a.block_tables, a.max_blocks_per_seq, a.context_lens, ctx_cap, a.num_seqs);
  return hipGetLastError();
}

}  // namespace pa
