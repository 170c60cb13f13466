// Slot-mapping scatter of new tokens' K and V into the paged KV pool.
//
// TensorSharp, Mistral 3 page, section 11 "Batched / paged forward": fresh
// K and V are written into the layer's paged buffer at
// blockId * blockSize + offset, with no per-sequence extract/inject.  The
// buffer's flat order [numBlocks, blockSize, numKvHeads, headDim] makes one
// slot's K (or V) for all kv heads one contiguous row of
// num_kv_heads * head_dim elements, so the scatter is a row copy.
//
// One thread moves one 16-byte chunk of K and the same chunk of V with
// 128-bit loads and stores; consecutive threads cover consecutive chunks of
// a row, so each row is read and written fully coalesced.  The copy moves
// bits and does no arithmetic, so it is exact for any element type.
#include "pa_common.h"

namespace pa {

__global__ void __launch_bounds__(256)
kv_cache_write_kernel(uint4 *__restrict__ k_cache, uint4 *__restrict__ v_cache, int64_t num_slots,
                      int chunks_per_row, const uint4 *__restrict__ key,
                      const uint4 *__restrict__ value, const int64_t *__restrict__ slots,
                      int num_tokens) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t token = gid / chunks_per_row;
  const int chunk = (int)(gid - token * chunks_per_row);
  if (token >= num_tokens) return;
  const int64_t slot = slots[token];
  if (slot < 0 || slot >= num_slots) return;  // padding, or outside the pool
  const int64_t src = token * chunks_per_row + chunk;
  const int64_t dst = slot * chunks_per_row + chunk;
  const uint4 kc = key[src];
  const uint4 vc = value[src];
  k_cache[dst] = kc;
  v_cache[dst] = vc;
}

hipError_t launch_kv_cache_write(void *k_cache, void *v_cache, int64_t num_slots, int row_bytes,
                                 const void *key, const void *value, const int64_t *slots,
                                 int num_tokens, hipStream_t stream) {
  const int chunks_per_row = row_bytes / 16;
  const int64_t total = (int64_t)num_tokens * chunks_per_row;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(kv_cache_write_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     static_cast<uint4 *>(k_cache), static_cast<uint4 *>(v_cache), num_slots,
                     chunks_per_row, static_cast<const uint4 *>(key),
                     static_cast<const uint4 *>(value), slots, num_tokens);
  return hipGetLastError();
}

// Whole-block copy between pools of the same block shape (or inside one
// pool): growing a pool into a larger allocation keeps the K/V of the
// sequences already placed (TensorSharp, Mistral 3 page, section 11, the
// grow path of the paged buffers), and a block-id map copies shared blocks
// for a sequence that must write into its own copy.  A block of K (or V) is
// block_size * num_kv_heads * head_dim contiguous elements; the grid walks
// 16-byte chunks of every (copy, K|V, block) with 128-bit loads and stores.
// Copies whose ids fall outside either pool are skipped.
__global__ void __launch_bounds__(256)
kv_cache_copy_blocks_kernel(const uint4 *__restrict__ src_k, const uint4 *__restrict__ src_v,
                            uint4 *__restrict__ dst_k, uint4 *__restrict__ dst_v, int src_blocks,
                            int dst_blocks, int64_t chunks_per_block, const int32_t *__restrict__ src_ids,
                            const int32_t *__restrict__ dst_ids, int num_copies) {
  const int64_t per_copy = 2 * chunks_per_block;  // K then V
  const int64_t total = (int64_t)num_copies * per_copy;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
       g += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = g / per_copy;
    int64_t r = g - c * per_copy;
    const bool is_v = r >= chunks_per_block;
    if (is_v) r -= chunks_per_block;
    const int sb = src_ids ? src_ids[c] : (int)c;
    const int db = dst_ids ? dst_ids[c] : (int)c;
    if ((unsigned)sb >= (unsigned)src_blocks || (unsigned)db >= (unsigned)dst_blocks) continue;
    const uint4 x = (is_v ? src_v : src_k)[(int64_t)sb * chunks_per_block + r];
    (is_v ? dst_v : dst_k)[(int64_t)db * chunks_per_block + r] = x;
  }
}

hipError_t launch_kv_cache_copy_blocks(const void *src_k, const void *src_v, void *dst_k, void *dst_v,
                                       int src_blocks, int dst_blocks, int64_t block_bytes,
                                       const int32_t *src_ids, const int32_t *dst_ids, int num_copies,
                                       hipStream_t stream) {
  const int64_t chunks = block_bytes / 16;
  const int64_t total = (int64_t)num_copies * 2 * chunks;
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;  // grid-stride beyond this
  hipLaunchKernelGGL(kv_cache_copy_blocks_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     static_cast<const uint4 *>(src_k), static_cast<const uint4 *>(src_v),
                     static_cast<uint4 *>(dst_k), static_cast<uint4 *>(dst_v), src_blocks, dst_blocks, chunks,
                     src_ids, dst_ids, num_copies);
  return hipGetLastError();
}

}  // namespace pa
