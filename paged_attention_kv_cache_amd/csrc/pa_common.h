// Internal helpers shared by the HIP kernels of the paged-attention library
// (gfx950 / CDNA4, wave64).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// ---------------------------------------------------------------- types
struct bf16_t {
  uint16_t bits;
};

template <typename T>
struct ElemTraits;
template <>
struct ElemTraits<float> {
  static constexpr int kBytes = 4;
};
template <>
struct ElemTraits<bf16_t> {
  static constexpr int kBytes = 2;
};

// bf16 <-> fp32.  Widening is exact (the bf16 bits are the high half of
// the fp32 bits); narrowing rounds to nearest, ties to even, and keeps NaN
// quiet.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;  // NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Widen a 16-byte chunk into floats.
template <typename T>
struct Chunk;
template <>
struct Chunk<float> {
  static constexpr int kElems = 4;
  __device__ __forceinline__ static void widen(const uint4 &c, float *f) {
    f[0] = __uint_as_float(c.x);
    f[1] = __uint_as_float(c.y);
    f[2] = __uint_as_float(c.z);
    f[3] = __uint_as_float(c.w);
  }
};
template <>
struct Chunk<bf16_t> {
  static constexpr int kElems = 8;
  __device__ __forceinline__ static void widen(const uint4 &c, float *f) {
    f[0] = bf16_lo(c.x);
    f[1] = bf16_hi(c.x);
    f[2] = bf16_lo(c.y);
    f[3] = bf16_hi(c.y);
    f[4] = bf16_lo(c.z);
    f[5] = bf16_hi(c.z);
    f[6] = bf16_lo(c.w);
    f[7] = bf16_hi(c.w);
  }
};

// N consecutive elements of T (N * sizeof(T) in {8, 16, 32} bytes, as
// aligned) loaded with 64- or 128-bit loads, then widened into floats.
template <typename T, int N>
struct Vec {
  static constexpr int kWords = N * ElemTraits<T>::kBytes / 4;
  static_assert(kWords == 2 || kWords == 4 || kWords == 8, "8, 16 or 32 bytes");
  uint32_t w[kWords];
  __device__ __forceinline__ void load(const T *p) {
    if constexpr (kWords == 2) {
      const uint2 c = *reinterpret_cast<const uint2 *>(p);
      w[0] = c.x, w[1] = c.y;
    } else {
#pragma unroll
      for (int i = 0; i < kWords / 4; ++i) {
        const uint4 c = reinterpret_cast<const uint4 *>(p)[i];
        w[4 * i] = c.x, w[4 * i + 1] = c.y, w[4 * i + 2] = c.z, w[4 * i + 3] = c.w;
      }
    }
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < kWords; ++i) w[i] = 0;
  }
  __device__ __forceinline__ void widen(float *f) const {
#pragma unroll
    for (int i = 0; i < kWords; ++i) {
      if constexpr (ElemTraits<T>::kBytes == 2) {
        f[2 * i] = bf16_lo(w[i]);
        f[2 * i + 1] = bf16_hi(w[i]);
      } else {
        f[i] = __uint_as_float(w[i]);
      }
    }
  }
};

// ------------------------------------------------------- lane exchanges
// DPP controls (GCN/CDNA encoding).
enum : int {
  kDppQuadXor1 = 0xB1,     // quad_perm [1,0,3,2]
  kDppQuadXor2 = 0x4E,     // quad_perm [2,3,0,1]
  kDppRowRor4 = 0x124,     // row_ror:4  (lane i reads lane (i+4) mod 16 of its row)
  kDppRowRor8 = 0x128,     // row_ror:8
  kDppRowHalfMirror = 0x141,
};

// Every control above reads a lane of the same row, so every lane gets a
// source value: no "old" value is needed (none is materialised), and the
// bound control (zero for a lane without a source) never applies; it lets
// the compiler fold the move into the instruction that uses it.
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, kCtrl, 0xF, 0xF, true);
}
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float x) {
  return __uint_as_float(dpp_u32<kCtrl>(__float_as_uint(x)));
}

// Sum over aligned groups of kLanes consecutive lanes (kLanes in
// {1,2,4,8,16,32,64}); every lane of the group receives the group sum.
template <int kLanes>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (kLanes >= 2) x += dpp_f32<kDppQuadXor1>(x);
  if constexpr (kLanes >= 4) x += dpp_f32<kDppQuadXor2>(x);
  if constexpr (kLanes == 8) x += dpp_f32<kDppRowHalfMirror>(x);
  if constexpr (kLanes >= 16) {
    x += dpp_f32<kDppRowRor4>(x);
    x += dpp_f32<kDppRowRor8>(x);
  }
  if constexpr (kLanes >= 32) x += __shfl_xor(x, 16);
  if constexpr (kLanes >= 64) x += __shfl_xor(x, 32);
  return x;
}

// Combine a value across the lanes that share (lane % kLanes), i.e. across
// the 64/kLanes groups of a wave.
template <int kLanes>
__device__ __forceinline__ float across_groups_max(float x) {
  if constexpr (kLanes <= 8) x = fmaxf(x, __shfl_xor(x, 8));
  if constexpr (kLanes <= 16) x = fmaxf(x, __shfl_xor(x, 16));
  if constexpr (kLanes <= 32) x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
template <int kLanes>
__device__ __forceinline__ float across_groups_sum(float x) {
  if constexpr (kLanes <= 8) x += __shfl_xor(x, 8);
  if constexpr (kLanes <= 16) x += __shfl_xor(x, 16);
  if constexpr (kLanes <= 32) x += __shfl_xor(x, 32);
  return x;
}

// gfx950 lane swaps: permlane16_swap(x, x) yields the even and the odd
// 16-lane row of each row pair, permlane32_swap(x, x) the two wave halves,
// so one VALU op plus an add combines lanes l and l^16 (or l^32).
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// bf16 pair helpers: fp32 dot product of two bf16 pairs plus an fp32
// addend (v_dot2_f32_bf16), and round-to-nearest-even packing of two floats
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;

}  // namespace pa

// ------------------------------------------------------------ launchers
// Host-side launchers implemented next to their kernels.  Arguments are
// already validated by the ABI layer.
namespace pa {

struct CacheView {
  const void *k;
  const void *v;
  int num_blocks, block_size, num_kv_heads, head_dim, dtype;
  int head_dim_v;  // value (and output) head dim
};

hipError_t launch_kv_cache_write(void *k_cache, void *v_cache, int64_t num_slots, int k_row_bytes,
                                 int v_row_bytes, const void *key, const void *value, const int64_t *slots,
                                 int num_tokens, hipStream_t stream);
hipError_t launch_kv_cache_copy_blocks(const void *src_k, const void *src_v, void *dst_k, void *dst_v,
                                       int src_blocks, int dst_blocks, int64_t k_block_bytes,
                                       int64_t v_block_bytes, const int32_t *src_ids, const int32_t *dst_ids,
                                       int num_copies, hipStream_t stream);

struct DecodeArgs {
  CacheView cache;
  void *out;
  const void *q;
  int num_seqs, num_heads;
  const int32_t *block_tables;
  int max_blocks_per_seq;
  const int32_t *context_lens;
  int max_context_len;
  float scale;
  int partition_size;      // > 0: tokens per partition (split-K); 0: single pass
  int max_partitions;      // ceil(max_context_len / partition_size), >= 1
  float *ws_m, *ws_l, *ws_o;
  // cascade decode (group_start non-NULL): rows group_start[g] ..
  // group_start[g+1]-1 share their first shared_len[g] tokens, whose
  // partials sit in slots 0 .. ceil(shared / shared_chunk) - 1 (one per
  // chunk); the partition launch computes those chunks once per group and
  // each row's own tokens into the following slots, and the reduce merges
  // every slot
  const int32_t *group_start = nullptr;
  const int32_t *shared_len = nullptr;
  int num_groups = 0;
  int shared_chunk = 64;   // the shared part's partials: slot c = tokens [c*chunk, (c+1)*chunk)
  int shared_cap = 0;      // shared tokens are clamped to this (shared_chunks * shared_chunk)
  int shared_chunks = 0;   // chunks per group the partition launch runs (cascade)
  int max_group_size = 0;  // rows of the largest group (cascade)
  // prefill rows (query_start_loc non-NULL; generic kernel, single pass):
  // "sequence" r is packed query row r of a chunked prefill over
  // num_prefill_seqs sequences; it reads the block table of the sequence
  // that owns it and sees that sequence's keys up to its own position
  const int32_t *query_start_loc = nullptr;
  int num_prefill_seqs = 0;
  // fused append (new_k non-NULL, bf16 matrix-core kernel only): the newest
  // token of each sequence (position context_len - 1) has its K and V rows
  // in new_k / new_v ([S, Hkv, D]) instead of the cache; the partition that
  // holds it attends to those rows and writes them into the token's slot
  const void *new_k = nullptr;
  const void *new_v = nullptr;
};

hipError_t launch_decode_partition(const DecodeArgs &a, hipStream_t stream);
// own-token partitions a cascade row may have, and the grid z extent of a
// cascade launch (its shared chunks and own partitions laid out over
// num_seqs x z)
int cascade_own_partitions(const DecodeArgs &a);
int cascade_grid_z(const DecodeArgs &a, int col_tiles);
// whether launch_decode_partition runs these shapes on the bf16
// matrix-core kernel (the one that can take the fused append)
bool decode_fast_path(const DecodeArgs &a);
// the cache write of a fused append, for the shapes the matrix-core kernel
// does not take: each sequence's new rows into the slot of its position
// context_len - 1 (through its block table); skipped for a context of 0 or
// a block id outside the pool
hipError_t launch_kv_cache_append(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_decode_reduce(const DecodeArgs &a, hipStream_t stream);

struct PrefillArgs {
  CacheView cache;
  void *out;
  const void *q;
  const int32_t *query_start_loc;
  int num_seqs, num_heads, num_query_tokens, max_query_len;
  const int32_t *block_tables;
  int max_blocks_per_seq;
  const int32_t *context_lens;
  int max_context_len;
  float scale;
};

hipError_t launch_prefill_chunk(const PrefillArgs &a, hipStream_t stream);

}  // namespace pa
