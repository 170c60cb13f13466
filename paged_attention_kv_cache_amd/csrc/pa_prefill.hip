// Chunked-prefill paged attention on bf16 MFMA tiles.
//
// What is computed: TensorSharp, Mistral 3 page, section 3 "Forward graph":
// scaled causal GQA attention of each new token over the cache, after the
// chunk's own K/V have been appended (pa_kv_cache_write runs first).  The
// chunk of a sequence sits at the end of its context: chunk row t has
// absolute position context_len - q_len + t and sees keys 0 .. that
// position.  Chunks of up to 512 tokens under a 4096-token budget are the
// shapes of the scheduling section of the mistral.rs comparison page.
//
// How it maps to gfx950:
//  * A work-group (4 waves) serves one kv head: its G query heads (4 at
//    most per work-group) x 32-token query groups of one sequence's chunk.
//    Every K/V tile is gathered once per work-group and shared by all of
//    its query heads through LDS.
//  * K/V tiles of 64 keys are gathered through the block table (one 16-byte
//    load per lane, whole rows coalesced) into LDS.  K is stored row-major
//    [key][d]; V is stored transposed [d][key].  Keys past the last
//    position the work-group needs, and keys in an invalid block, are
//    zero-filled, so a masked key never brings a NaN into the products.
//  * Scores are computed transposed, S^T = K Q^T, on
//    v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q^T held in registers).
//    In the accumulator layout every lane then holds 16 keys of one query,
//    so the online-softmax max and sum need one cross-half exchange only,
//    and the rescale factor is a per-lane scalar.
//  * The weights, rounded to bf16, are already in the B-operand layout of
//    O^T += V^T P^T (A = V^T from LDS), so P never goes through LDS.
//  * The causal mask (bottom-right aligned) is applied only on tiles that
//    cross the diagonal of the wave's 32 queries, by selecting -inf.
//  * Work ids are remapped so that the query tiles of one (sequence, kv
//    head), which read the same K/V, land on the same XCD and share its L2.
//    Tiles with more keys (later in the chunk) are dispatched first.
#include "pa_common.h"

namespace pa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

struct PrefillKernelArgs {
  void *out;
  const void *q;
  const void *k_cache;
  const void *v_cache;
  const int32_t *query_start_loc;
  const int32_t *block_tables;
  const int32_t *context_lens;
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int num_blocks;
  int block_shift;
  int max_blocks_per_seq;
  int ctx_cap;            // min(max_context_len, max_blocks_per_seq * block_size)
  int num_query_tokens;
  int n_qtiles;           // query tiles per (sequence, head group)
  int n_work;             // work-groups with work
  float scale_log2;       // scale * log2(e)
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ bf16x8_t pack8(const f32x16_t &s, int base) {
  bf16x8_t r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)s[base + e];
  return r;
}

template <int D, int G>
__global__ void __launch_bounds__(256)
prefill_chunk_kernel(const PrefillKernelArgs a) {
  constexpr int GW = G < 4 ? G : 4;  // query heads per work-group
  constexpr int HALVES = G / GW;     // work-groups per kv head along heads
  constexpr int TG = 4 / GW;         // 32-token query groups per work-group
  constexpr int QT = 32 * TG;        // query tokens per work-group
  constexpr int KT = 64;             // keys per tile
  constexpr int KSTR = D + 8;        // LDS row stride of K, bf16 elements
  constexpr int VSTR = KT + 8;       // LDS row stride of V^T, bf16 elements
  constexpr int NDS = D / 16;        // k-steps of Q K^T
  constexpr int NDT = D / 32;        // 32-row tiles of O^T
  constexpr int C16 = D / 8;         // 16-byte chunks per K/V row

  __shared__ __attribute__((aligned(16))) uint16_t sk[KT * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t svt[D * VSTR];

  // work id: consecutive ids share a (sequence, kv head) and sit on one XCD
  const int nwg = gridDim.x;  // a multiple of 8
  const int bid = blockIdx.x;
  const int wid = (bid & 7) * (nwg >> 3) + (bid >> 3);
  if (wid >= a.n_work) return;
  int rest = wid;
  const int qt_rev = rest % a.n_qtiles;
  rest /= a.n_qtiles;
  const int half = rest % HALVES;
  rest /= HALVES;
  const int kvh = rest % a.num_kv_heads;
  const int seq = rest / a.num_kv_heads;
  const int qtile = a.n_qtiles - 1 - qt_rev;

  int r1 = min(a.query_start_loc[seq + 1], a.num_query_tokens);
  int r0 = a.query_start_loc[seq];
  r0 = max(0, min(r0, r1));
  const int q_len = r1 - r0;
  int ctx = min(a.context_lens[seq], a.ctx_cap);
  ctx = max(ctx, 0);
  const int t_begin = qtile * QT;
  if (t_begin >= q_len) return;
  const int prefix = ctx - q_len;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hl = wave % GW;
  const int tg = wave / GW;
  const int head = kvh * G + half * GW + hl;
  const int tw0 = t_begin + tg * 32;  // first query of this wave
  const int col = lane & 31;
  const int hh = lane >> 5;
  const int t = tw0 + col;            // this lane's query (chunk row)
  const bool qvalid = t < q_len;
  const int qpos = prefix + t;

  bf16x8_t qb[NDS];
  {
    const uint4 *qrow = reinterpret_cast<const uint4 *>(
        static_cast<const uint16_t *>(a.q) + ((size_t)(r0 + (qvalid ? t : 0)) * a.num_heads + head) * D);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) qb[ds] = as_bf16x8(qvalid ? qrow[ds * 2 + hh] : make_uint4(0, 0, 0, 0));
  }

  // keys this work-group needs: 0 .. (largest query position of the tile)
  const int t_last = min(t_begin + QT, q_len) - 1;
  const int kend = max(0, min(ctx, prefix + t_last + 1));
  const int ntiles = (kend + KT - 1) / KT;

  const size_t slot_stride = (size_t)a.num_kv_heads * D;
  const uint16_t *kbase = static_cast<const uint16_t *>(a.k_cache) + (size_t)kvh * D;
  const uint16_t *vbase = static_cast<const uint16_t *>(a.v_cache) + (size_t)kvh * D;
  const int32_t *bt = a.block_tables + (size_t)seq * a.max_blocks_per_seq;
  const int shift = a.block_shift;
  const int bs_mask = (1 << shift) - 1;
  const float sl = a.scale_log2;

  float m = -INFINITY;  // running max of this lane's query (base-2 units)
  float l = 0.f;        // running sum over this lane's keys
  f32x16_t o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;

  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * KT;
    // K tile, row-major: C16 lanes per key row, whole rows coalesced
#pragma unroll
    for (int j = 0; j < KT * C16 / 256; ++j) {
      const int i = tid + 256 * j;
      const int key = i / C16;
      const int c = i % C16;
      const int kpos = k0 + key;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (kpos < kend) {
        const int blk = bt[kpos >> shift];
        if ((unsigned)blk < (unsigned)a.num_blocks)
          val = *reinterpret_cast<const uint4 *>(
              kbase + ((size_t)(blk << shift) + (size_t)(kpos & bs_mask)) * slot_stride + c * 8);
      }
      *reinterpret_cast<uint4 *>(sk + key * KSTR + c * 8) = val;
    }
    // V tile, transposed: a lane takes keys 2p and 2p+1 of one 16-byte
    // column chunk and writes (V[2p][d], V[2p+1][d]) pairs as dwords
#pragma unroll
    for (int j = 0; j < 32 * C16 / 256; ++j) {
      const int i = tid + 256 * j;
      const int p = i % 32;
      const int c = i / 32;
      const int ka = k0 + 2 * p;
      uint4 va = make_uint4(0, 0, 0, 0), vb = make_uint4(0, 0, 0, 0);
      if (ka < kend) {
        const int blk = bt[ka >> shift];
        if ((unsigned)blk < (unsigned)a.num_blocks)
          va = *reinterpret_cast<const uint4 *>(
              vbase + ((size_t)(blk << shift) + (size_t)(ka & bs_mask)) * slot_stride + c * 8);
      }
      if (ka + 1 < kend) {
        const int blk = bt[(ka + 1) >> shift];
        if ((unsigned)blk < (unsigned)a.num_blocks)
          vb = *reinterpret_cast<const uint4 *>(
              vbase + ((size_t)(blk << shift) + (size_t)((ka + 1) & bs_mask)) * slot_stride + c * 8);
      }
      uint32_t *dst = reinterpret_cast<uint32_t *>(svt + (c * 8) * VSTR + 2 * p);
      constexpr int kRowWords = VSTR / 2;
      dst[0 * kRowWords] = interleave_lo(va.x, vb.x);
      dst[1 * kRowWords] = interleave_hi(va.x, vb.x);
      dst[2 * kRowWords] = interleave_lo(va.y, vb.y);
      dst[3 * kRowWords] = interleave_hi(va.y, vb.y);
      dst[4 * kRowWords] = interleave_lo(va.z, vb.z);
      dst[5 * kRowWords] = interleave_hi(va.z, vb.z);
      dst[6 * kRowWords] = interleave_lo(va.w, vb.w);
      dst[7 * kRowWords] = interleave_hi(va.w, vb.w);
    }
    __syncthreads();

    // S^T = K Q^T for keys k0 .. k0+31 (s0) and k0+32 .. k0+63 (s1)
    f32x16_t s0, s1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = 0.f;
      s1[r] = 0.f;
    }
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t *>(sk + col * KSTR + ds * 16 + hh * 8);
      const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t *>(sk + (32 + col) * KSTR + ds * 16 + hh * 8);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qb[ds], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qb[ds], s1, 0, 0, 0);
    }

    // scale; causal mask on tiles that cross this wave's diagonal.
    // Accumulator register r of this lane holds key 8*(r/4) + 4*hh + r%4.
    const bool diag = k0 + KT - 1 > prefix + tw0;
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = 8 * (r >> 2) + 4 * hh + (r & 3);
      float v0 = s0[r] * sl;
      float v1 = s1[r] * sl;
      if (diag) {
        v0 = (k0 + kr <= qpos) ? v0 : -INFINITY;
        v1 = (k0 + 32 + kr <= qpos) ? v1 : -INFINITY;
      }
      s0[r] = v0;
      s1[r] = v1;
      tmax = fmaxf(tmax, fmaxf(v0, v1));
    }
    tmax = xor32_max(tmax);
    const float m_new = fmaxf(m, tmax);
    const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m - m_new);
    m = m_new;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p0 = (m == -INFINITY) ? 0.f : fast_exp2(s0[r] - m);
      const float p1 = (m == -INFINITY) ? 0.f : fast_exp2(s1[r] - m);
      s0[r] = p0;
      s1[r] = p1;
      psum += p0 + p1;
    }
    l = l * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;

    // P^T in the B layout: k-step (sub-tile st, half u) = registers 8u..8u+7
    // of s_st, i.e. keys st*32 + 16u + 8*(e/4) + 4*hh + e%4 for slot e
    bf16x8_t pb[4];
    pb[0] = pack8(s0, 0);
    pb[1] = pack8(s0, 8);
    pb[2] = pack8(s1, 0);
    pb[3] = pack8(s1, 8);

    // O^T += V^T P^T; the A operand takes the same keys from row d of V^T
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const uint16_t *vrow = svt + (dt * 32 + col) * VSTR;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kb0 = (ks >> 1) * 32 + (ks & 1) * 16 + 4 * hh;
        const uint2 lo = *reinterpret_cast<const uint2 *>(vrow + kb0);
        const uint2 hi = *reinterpret_cast<const uint2 *>(vrow + kb0 + 8);
        const bf16x8_t av = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[ks], o[dt], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  const float lt = xor32_sum(l);
  if (qvalid) {
    uint16_t *orow = static_cast<uint16_t *>(a.out) + ((size_t)(r0 + t) * a.num_heads + head) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = dt * 32 + 8 * rq + 4 * hh;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (lt > 0.f) ? o[dt][4 * rq + e] / lt : 0.f;
        *reinterpret_cast<uint2 *>(orow + d0) = make_uint2(pack_bf16x2_rne(v[0], v[1]), pack_bf16x2_rne(v[2], v[3]));
      }
  }
}

template <int D, int G>
static hipError_t launch_t(const PrefillArgs &a, hipStream_t stream) {
  constexpr int GW = G < 4 ? G : 4;
  constexpr int HALVES = G / GW;
  constexpr int QT = 32 * (4 / GW);
  PrefillKernelArgs k;
  k.out = a.out;
  k.q = a.q;
  k.k_cache = a.cache.k;
  k.v_cache = a.cache.v;
  k.query_start_loc = a.query_start_loc;
  k.block_tables = a.block_tables;
  k.context_lens = a.context_lens;
  k.num_seqs = a.num_seqs;
  k.num_heads = a.num_heads;
  k.num_kv_heads = a.cache.num_kv_heads;
  k.num_blocks = a.cache.num_blocks;
  int shift = 0;
  while ((1 << shift) < a.cache.block_size) ++shift;
  k.block_shift = shift;
  k.max_blocks_per_seq = a.max_blocks_per_seq;
  const int64_t table_cap = (int64_t)a.max_blocks_per_seq * a.cache.block_size;
  k.ctx_cap = (int)(table_cap < a.max_context_len ? table_cap : a.max_context_len);
  k.num_query_tokens = a.num_query_tokens;
  k.n_qtiles = (a.max_query_len + QT - 1) / QT;
  const int64_t n_work = (int64_t)a.num_seqs * a.cache.num_kv_heads * HALVES * k.n_qtiles;
  if (n_work <= 0) return hipSuccess;
  if (n_work > (int64_t)0x7fffffff - 8) return hipErrorInvalidConfiguration;
  k.n_work = (int)n_work;
  k.scale_log2 = a.scale * kLog2e;
  const unsigned grid = (unsigned)((n_work + 7) / 8 * 8);
  hipLaunchKernelGGL((prefill_chunk_kernel<D, G>), dim3(grid), dim3(256), 0, stream, k);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_g(const PrefillArgs &a, hipStream_t stream) {
  switch (a.num_heads / a.cache.num_kv_heads) {
    case 1: return launch_t<D, 1>(a, stream);
    case 2: return launch_t<D, 2>(a, stream);
    case 4: return launch_t<D, 4>(a, stream);
    case 8: return launch_t<D, 8>(a, stream);
  }
  return hipErrorNotSupported;
}

hipError_t launch_prefill_chunk(const PrefillArgs &a, hipStream_t stream) {
  if (a.cache.dtype != 1) return hipErrorNotSupported;
  switch (a.cache.head_dim) {
    case 64: return launch_g<64>(a, stream);
    case 128: return launch_g<128>(a, stream);
  }
  return hipErrorNotSupported;
}

}  // namespace pa
