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
//  * A work-group (8 waves) serves one kv head: its G query heads (8 at
//    most) x 32-token query groups of one sequence's chunk (64 tokens for
//    G = 4).
//    Every K/V tile is gathered once per work-group and shared by all of
//    its query heads through LDS.
//  * K/V tiles of 64 keys are gathered through the block table straight
//    into LDS with 16-byte global-to-LDS loads (no registers, no LDS store
//    instructions), both row-major [key][d] in swizzled 64-byte chunk
//    groups (see TileGather).  Keys past the last position the work-group
//    needs, and keys in an invalid block, read a zero chunk instead, so a
//    masked key never brings a NaN into the products.
//  * Scores are computed transposed, S^T = K Q^T, on
//    v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q^T held in registers).
//    In the accumulator layout every lane then holds 16 keys of one query,
//    so the online-softmax max and sum need one cross-half exchange only,
//    and the rescale factor is a per-lane scalar.
//  * The weights, rounded to bf16, are already in the B-operand layout of
//    O^T += V^T P^T, so P never goes through LDS; the A operand (V^T) comes
//    from the row-major V tile through gfx950's transposing LDS reads.
//  * The causal mask (bottom-right aligned) is applied only on tiles that
//    cross the diagonal of the wave's 32 queries, by selecting -inf.
//  * LDS holds three K and three V tiles.  In step t a wave computes the
//    scores of tile t+1 while it runs the softmax of tile t (independent
//    work for the matrix and vector units), then multiplies V of tile t;
//    the loads of tile t+2 into LDS are in flight meanwhile and are waited
//    for before the step's single barrier.
//  * The output is rescaled only when a query's max grows by more than 2^8
//    (the final division by the running sum makes any reference max exact).
//  * Work ids are remapped so that each XCD serves whole kv heads of every
//    sequence: the XCDs get equal work, and the query tiles of one
//    (sequence, kv head), which read the same K/V, share that XCD's L2.
//    Within a kv head the (sequence, query tile) items are dispatched
//    longest first (most keys to read).
//  * Key and value head dims may differ (section 4.1 of the same page):
//    the K tile, Q and the score products take the key dim D, the V^T tile
//    and the output tiles the value dim DV.
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
  // shared-prefix pass of cascade decode (group_start non-NULL): a "sequence"
  // is a group of decode rows group_start[g] .. group_start[g+1]-1 whose
  // first shared_len[g] tokens are the same blocks; their attention over
  // those tokens is written as split-K partials into slot 0 of ws_*
  const int32_t *group_start;
  const int32_t *shared_len;
  float *ws_m;
  float *ws_l;
  float *ws_o;
  int ws_parts;           // partition slots per (row, head)
  int n_chunks;           // key chunks per group (1 for prefill)
  int chunk;              // tokens per key chunk, a multiple of 64 (cascade)
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ bf16x8_t pack8(const f32x16_t &s, int base) {
  bf16x8_t r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)s[base + e];
  return r;
}

// waves per work-group (8: one work-group per CU shares each tile among
// 8 waves; 4: two work-groups per CU, whose phases drift apart)
#ifndef PA_PREFILL_WAVES
#define PA_PREFILL_WAVES 8
#endif
constexpr int kPrefillThreads = 64 * PA_PREFILL_WAVES;
// query heads per wave (1 or 2); with 2, each K and V^T fragment read from
// LDS feeds two MFMAs
#ifndef PA_PREFILL_HW
#define PA_PREFILL_HW 1
#endif
// 1: a wave computes the scores of tile t+1 while it runs the softmax of
// tile t (costs a second set of score registers); 0: the scores of tile t
// at the start of step t (with two heads per wave, one head's products
// overlap the other head's softmax)
#ifndef PA_PREFILL_LOOKAHEAD
#define PA_PREFILL_LOOKAHEAD (PA_PREFILL_HW == 1)
#endif
#ifndef PA_PREFILL_ORDER
#define PA_PREFILL_ORDER 1
#endif
// 1: within each (kv head, head part), the (sequence, query tile) items of
// a batch with at most 64 of them are dispatched longest first (keys to
// read, largest first), the classic longest-processing-time order; larger
// batches and cascade launches keep the plain order
#ifndef PA_PREFILL_LPT
#define PA_PREFILL_LPT 1
#endif

constexpr int kMaxTileBlocks = 8;  // 64 keys / smallest block size

// block ids of the tile starting at key k0 (64 / block_size entries); the
// work-group keeps them in a tiny LDS array, filled ahead of time
__device__ __forceinline__ int tile_block_id(const int32_t *bt, int k0, int j, int shift, int max_blocks) {
  return bt[min((k0 >> shift) + j, max_blocks - 1)];
}

typedef __attribute__((address_space(3))) void *lds_ptr_t;

// source of the 16-byte chunks of keys that must read as zero
__device__ const uint4 kZeroChunk = {0u, 0u, 0u, 0u};

// Gather of one K (or V) tile, keys k0 .. k0+63 of row width DIM, straight
// from the pool into LDS with 16-byte global-to-LDS loads: no registers, no
// LDS store instructions.  LDS layout: the row's 16-byte chunks in groups of
// four (64 bytes, 32 elements): group g of every key forms a 4 KB block
// [key][4 chunks], and inside a key's 64 bytes chunk c sits in slot
// (c % 4) ^ ((k / 4) % 4).  Sixteen consecutive keys then cover all LDS
// banks for any fixed chunk, and the slot pattern depends on a lane's key
// only through (k / 4) % 4, so every fragment read is a per-lane base plus
// a compile-time offset.  A wave's load writes 1 KB of consecutive LDS
// (lane i at 16 i): 16 keys x one chunk group, each lane fetching the global
// chunk that belongs in its slot.  A tile starts at a multiple of 64 keys
// and the block size divides 64, so a lane's key, its block's index in the
// tile and its offset inside the block are the same for every tile; only
// the block ids change.  A key at or past kend, or in a block outside the
// pool, reads a 16-byte zero chunk instead, so its K and V rows are zero.
template <int DIM>
struct TileGather {
  static constexpr int CG = DIM / 32;                              // chunk groups per row
  static constexpr int CPR = DIM / 8;                              // 16-byte chunks per row
  static constexpr int PER_WAVE = (CG * 4) / (kPrefillThreads / 64);  // wave loads per tile
  static_assert(PER_WAVE >= 1 && (CG * 4) % (kPrefillThreads / 64) == 0, "tile split over the waves");
  int key[PER_WAVE];        // this lane's key inside the tile, per load
  uint32_t off[PER_WAVE];   // element offset inside the block (row, head, chunk)
  uint32_t lds[PER_WAVE];   // byte offset of the wave's load inside the tile (wave-uniform)

  __device__ __forceinline__ void init(int wave, int lane, int shift, int bs_mask, uint32_t slot_stride) {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int load = wave * PER_WAVE + j;  // chunk group load / 4, key group load % 4
      const int key = (load % 4) * 16 + lane / 4;
      const int chunk = (load / 4) * 4 + ((lane % 4) ^ ((key >> 2) & 3));
      this->key[j] = key;
      off[j] = (uint32_t)(key & bs_mask) * slot_stride + (uint32_t)chunk * 8;
      lds[j] = (uint32_t)load * 1024;
    }
  }
  __device__ __forceinline__ void issue(uint16_t *tile, const int *ids, const uint16_t *base, int num_blocks,
                                        size_t block_stride, int k0, int kend, int shift) const {
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
      const int b = ids[key[j] >> shift];
      const bool ok = (unsigned)b < (unsigned)num_blocks && k0 + key[j] < kend;
      const void *src = ok ? static_cast<const void *>(base + (size_t)b * block_stride + off[j])
                           : static_cast<const void *>(&kZeroChunk);
      __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(reinterpret_cast<char *>(tile) + lds[j]), 16, 0, 0);
    }
  }
};

// a rescale of O is done only when a query's running max grows by more than
// this many base-2 units; until then the weights may exceed 1 by up to 2^8,
// which the fp32 accumulators and the bf16 weights carry exactly as well
constexpr float kRescaleSlack = 8.f;

constexpr uint32_t kBf16PairOnes = 0x3F803F80u;  // two bf16 1.0

template <int G>
struct PrefillShape {
  static constexpr int NW = kPrefillThreads / 64;  // waves per work-group
  static constexpr int HW = (G >= 2) ? PA_PREFILL_HW : 1;  // query heads per wave
  static constexpr int HP = G / HW;                // head slots of a kv head
  static constexpr int GWH = HP < NW ? HP : NW;    // head slots per work-group
  static constexpr int HALVES = HP / GWH;          // work-groups per kv head along heads
  static constexpr int TG = NW / GWH;              // 32-token query groups per work-group
  static constexpr int QT = 32 * TG;               // query tokens per work-group
  static_assert(HP % GWH == 0 && NW % GWH == 0, "heads and waves must divide");
};

template <int D, int DV, int G>
__global__ void __launch_bounds__(kPrefillThreads, (8 / PA_PREFILL_WAVES) / PA_PREFILL_HW)
prefill_chunk_kernel(const PrefillKernelArgs a) {
  using Sh = PrefillShape<G>;
  constexpr int HW = Sh::HW;
  constexpr int GWH = Sh::GWH;
  constexpr int HALVES = Sh::HALVES;
  constexpr int QT = Sh::QT;
  constexpr int KT = 64;             // keys per tile
  using GK = TileGather<D>;
  using GV = TileGather<DV>;
  constexpr int NDS = D / 16;        // k-steps of Q K^T
  constexpr int NDT = DV / 32;       // 32-row tiles of O^T

  // three buffers each for K and V: at step t the waves read K of tile t+1
  // and V of tile t while tile t+2 is loaded
  __shared__ __attribute__((aligned(1024))) uint16_t sk[3][KT * D];
  __shared__ __attribute__((aligned(1024))) uint16_t sv[3][KT * DV];
  __shared__ int sid[3][kMaxTileBlocks];

  // Work id.  Work-groups are dispatched round-robin over the 8 XCDs; the
  // remap gives each XCD a contiguous range of work ids, ordered (kv head,
  // head part, sequence, query tile from the last): the query tiles of one
  // (sequence, kv head), which read the same K/V, run together on one XCD
  // and share its L2, the tiles with more keys first.
  const int nwg = gridDim.x;  // a multiple of 8
  const int bid = blockIdx.x;
  const int wid = (bid & 7) * (nwg >> 3) + (bid >> 3);
  if (wid >= a.n_work) return;
  int rest = wid;
  const int kchunk = rest % a.n_chunks;  // cascade: chunk of the shared tokens
  rest /= a.n_chunks;
#if PA_PREFILL_ORDER == 1
  const int qt_rev = rest % a.n_qtiles;
  rest /= a.n_qtiles;
  const int seq0 = rest % a.num_seqs;
  rest /= a.num_seqs;
#else
  const int seq0 = rest % a.num_seqs;
  rest /= a.num_seqs;
  const int qt_rev = rest % a.n_qtiles;
  rest /= a.n_qtiles;
#endif
  const int half = rest % HALVES;
  const int kvh = rest / HALVES;
  int qtile = a.n_qtiles - 1 - qt_rev;
  const bool cascade = a.group_start != nullptr;
#if PA_PREFILL_LPT && PA_PREFILL_ORDER == 1
  int seq = seq0;
  if (!cascade && a.num_seqs * a.n_qtiles <= 64) {
    // item j of this (kv head, head part) takes the j-th largest item: lane
    // i of wave 0 holds item i = (sequence i / n_qtiles, query tile
    // i % n_qtiles) and its key-tile count, ranked by (count descending,
    // index ascending)
    __shared__ int s_item;
    if (threadIdx.x < 64) {
      const int i = threadIdx.x;
      const int n_items = a.num_seqs * a.n_qtiles;
      int work = -1;  // past the items: ranked after every item
      if (i < n_items) {
        const int sq = i / a.n_qtiles;
        const int qt = i - sq * a.n_qtiles;
        const int e1 = min(a.query_start_loc[sq + 1], a.num_query_tokens);
        const int e0 = max(0, min(a.query_start_loc[sq], e1));
        const int ql = e1 - e0;
        const int c = max(0, min(a.context_lens[sq], a.ctx_cap));
        work = 0;
        if (qt * QT < ql) {
          const int tl = min(qt * QT + QT, ql) - 1;
          const int ke = max(0, min(c, c - ql + tl + 1));
          work = (ke + KT - 1) / KT + 1;  // key tiles, plus about one tile of fixed cost
        }
      }
      int rank = 0;
      for (int k = 0; k < 64; ++k) {
        const int wk = __builtin_amdgcn_readlane(work, k);
        rank += (wk > work || (wk == work && k < i)) ? 1 : 0;
      }
      const int j = seq0 * a.n_qtiles + qt_rev;
      const unsigned long long hit = __builtin_amdgcn_ballot_w64(i < n_items && rank == j);
      if (i == 0) s_item = hit ? (int)__builtin_ctzll(hit) : 0;
    }
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(s_item);
    seq = item / a.n_qtiles;
    qtile = item - seq * a.n_qtiles;
  }
#else
  const int seq = seq0;
#endif

  const int32_t *rows = cascade ? a.group_start : a.query_start_loc;
  int r1 = min(rows[seq + 1], a.num_query_tokens);
  int r0 = rows[seq];
  r0 = max(0, min(r0, r1));
  const int q_len = r1 - r0;
  // prefill: the chunk ends the context; cascade: the shared tokens
  int ctx = min(cascade ? min(a.shared_len[seq], a.n_chunks * a.chunk) : a.context_lens[seq], a.ctx_cap);
  ctx = max(ctx, 0);
  const int t_begin = qtile * QT;
  if (t_begin >= q_len) return;
  if (cascade && kchunk * a.chunk >= ctx) return;  // a chunk past the group's shared tokens
  const int prefix = ctx - q_len;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hs = wave % GWH;           // head slot of this wave
  const int tg = wave / GWH;
  const int head0 = kvh * G + (half * GWH + hs) * HW;  // first of the wave's HW heads
  const int tw0 = t_begin + tg * 32;   // first query of this wave
  const int col = lane & 31;
  const int hh = lane >> 5;
  const int t = tw0 + col;             // this lane's query (chunk row)
  const bool qvalid = t < q_len;
  // last key this lane's query sees: its chunk position (prefill), or the
  // end of the shared tokens within the row's own context (cascade)
  int qpos = prefix + t;
  if (cascade) {
    const int own = qvalid ? max(0, min(a.context_lens[r0 + t], a.ctx_cap)) : ctx;
    qpos = min(ctx, own) - 1;
  }
  // smallest of them in the wave: tiles past it need the mask
  int qpos_lo = qpos;
#pragma unroll
  for (int sft = 1; sft < 64; sft <<= 1) qpos_lo = min(qpos_lo, __shfl_xor(qpos_lo, sft));
  qpos_lo = __builtin_amdgcn_readfirstlane(qpos_lo);

  bf16x8_t qb[HW][NDS];
#pragma unroll
  for (int h = 0; h < HW; ++h) {
    const uint4 *qrow = reinterpret_cast<const uint4 *>(
        static_cast<const uint16_t *>(a.q) + ((size_t)(r0 + (qvalid ? t : 0)) * a.num_heads + head0 + h) * D);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) qb[h][ds] = as_bf16x8(qvalid ? qrow[ds * 2 + hh] : make_uint4(0, 0, 0, 0));
  }

  // keys this work-group needs: 0 .. (largest query position of the tile)
  const int t_last = min(t_begin + QT, q_len) - 1;
  int kend = max(0, min(ctx, prefix + t_last + 1));
  // cascade: the shared blocks are read through the table of the group's
  // longest row, up to min(shared, its context), so every key read lies in
  // a real context (a shorter row masks the keys it does not have)
  int tab_row = seq;
  if (cascade) {
    __shared__ int s_best[2];
    if (wave == 0) {
      int best = -1, brow = r0;
      for (int i = r0 + lane; i < r1; i += 64) {
        const int c = max(0, min(a.context_lens[i], a.ctx_cap));
        if (c > best) {
          best = c;
          brow = i;
        }
      }
#pragma unroll
      for (int sft = 1; sft < 64; sft <<= 1) {
        const int ob = __shfl_xor(best, sft);
        const int orow = __shfl_xor(brow, sft);
        if (ob > best || (ob == best && orow < brow)) {
          best = ob;
          brow = orow;
        }
      }
      if (lane == 0) {
        s_best[0] = best;
        s_best[1] = brow;
      }
    }
    __syncthreads();
    kend = max(0, min(ctx, s_best[0]));
    tab_row = s_best[1];
  }
  // cascade: this work-group's chunk of the shared tokens
  const int kbeg = cascade ? kchunk * a.chunk : 0;
  if (cascade) {
    kend = min(kend, kbeg + a.chunk);
    if (kbeg >= kend) return;  // past every row's shared tokens: a slot no merge reads
  }

  const uint32_t slot_stride = (uint32_t)a.num_kv_heads * D;  // elements between K slots
  const uint32_t vslot_stride = (uint32_t)a.num_kv_heads * DV;
  const size_t block_stride = (size_t)slot_stride << a.block_shift;
  const size_t vblock_stride = (size_t)vslot_stride << a.block_shift;
  const uint16_t *kbase = static_cast<const uint16_t *>(a.k_cache) + (size_t)kvh * D;
  const uint16_t *vbase = static_cast<const uint16_t *>(a.v_cache) + (size_t)kvh * DV;
  const int32_t *bt = a.block_tables + (size_t)tab_row * a.max_blocks_per_seq;
  const int shift = a.block_shift;
  const int bs_mask = (1 << shift) - 1;
  const float sl = a.scale_log2;
  GK gk;
  GV gv;
  gk.init(wave, lane, shift, bs_mask, slot_stride);
  gv.init(wave, lane, shift, bs_mask, vslot_stride);
  // per-lane parts of the fragment addresses (see TileGather)
  const int k_even = ((hh ^ ((col >> 2) & 3)) << 4);
  const int k_odd = (((2 + hh) ^ ((col >> 2) & 3)) << 4);
  const int vg = lane >> 4, vs = lane & 15;
  const int v_lane = (4 * (vg >> 1) + (vs >> 2)) * 64 + (vs & 1) * 8;
  const int v_slot = 2 * (vg & 1) + ((vs >> 1) & 1);
  const int v_off0 = v_lane + ((v_slot ^ ((vg >> 1) & 3)) << 4);        // keys of the first read
  const int v_off1 = v_lane + 8 * 64 + ((v_slot ^ (((vg >> 1) + 2) & 3)) << 4);  // 8 keys further

  float m[HW], l[HW];  // reference max (base-2 units) and running sum of this lane's query, per head
  f32x16_t o[HW][NDT];
#pragma unroll
  for (int h = 0; h < HW; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[h][dt][r] = 0.f;
  }

  // S^T tiles of keys k0 .. k0+63 for the wave's heads (s0: first 32 keys,
  // s1: last 32); each K fragment read from LDS feeds HW products
  auto qk = [&](const uint16_t *skb, f32x16_t (&s0)[HW], f32x16_t (&s1)[HW]) {
#pragma unroll
    for (int h = 0; h < HW; ++h)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s0[h][r] = 0.f;
        s1[h][r] = 0.f;
      }
    // chunk 2 ds + hh of keys col and 32 + col: group ds / 2, slot
    // (2 (ds % 2) + hh) ^ ((col / 4) % 4)
    typedef __attribute__((address_space(3))) const char *lds_cptr;
    typedef __attribute__((address_space(3))) const bf16x8_t *lds_frag_ptr;
    uint32_t ke = (uint32_t)(size_t)((lds_cptr)(const char *)skb + col * 64 + k_even);
    uint32_t ko = (uint32_t)(size_t)((lds_cptr)(const char *)skb + col * 64 + k_odd);
    asm volatile("" : "+v"(ke), "+v"(ko));
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const uint32_t p = ((ds & 1) ? ko : ke) + (ds / 2) * 4096;
      const bf16x8_t a0 = *(lds_frag_ptr)(size_t)(p);
      const bf16x8_t a1 = *(lds_frag_ptr)(size_t)(p + 2048);
#pragma unroll
      for (int h = 0; h < HW; ++h) {
        s0[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qb[h][ds], s0[h], 0, 0, 0);
        s1[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qb[h][ds], s1[h], 0, 0, 0);
      }
    }
  };

  // Pipeline, one barrier per step t:
  //   global-to-LDS loads of tile t+2 issued;  S(t+1) = K(t+1) Q^T;
  //   softmax of S(t);  O += V(t) P(t);  wait for this wave's loads.
  // Block ids: sid[j % 3] holds the ids of tile j, filled three tiles ahead.
  if (tid < kMaxTileBlocks) {
#pragma unroll
    for (int j = 0; j < 3; ++j) sid[j][tid] = tile_block_id(bt, kbeg + j * KT, tid, shift, a.max_blocks_per_seq);
  }
  __syncthreads();
  const int ntiles = (kend - kbeg + KT - 1) / KT;
  gk.issue(sk[0], sid[0], kbase, a.num_blocks, block_stride, kbeg, kend, shift);
  gv.issue(sv[0], sid[0], vbase, a.num_blocks, vblock_stride, kbeg, kend, shift);
  gk.issue(sk[1], sid[1], kbase, a.num_blocks, block_stride, kbeg + KT, kend, shift);
  gv.issue(sv[1], sid[1], vbase, a.num_blocks, vblock_stride, kbeg + KT, kend, shift);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  f32x16_t c0[HW], c1[HW];  // S of the current tile
#if PA_PREFILL_LOOKAHEAD
  qk(sk[0], c0, c1);
#endif

  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kbeg + kt * KT;
    const int b0 = kt % 3;
    const int b1 = (kt + 1) % 3;
    const int b2 = (kt + 2) % 3;
#if !PA_PREFILL_LOOKAHEAD
    qk(sk[b0], c0, c1);
#endif
    // tile t+2 from the pool (past the last tile: zero rows, never used)
    gk.issue(sk[b2], sid[b2], kbase, a.num_blocks, block_stride, k0 + 2 * KT, kend, shift);
    gv.issue(sv[b2], sid[b2], vbase, a.num_blocks, vblock_stride, k0 + 2 * KT, kend, shift);
    int next_id = 0;
    if (tid < kMaxTileBlocks) next_id = tile_block_id(bt, k0 + 3 * KT, tid, shift, a.max_blocks_per_seq);

    // causal mask on tiles that cross this wave's diagonal (raw scores;
    // register r of this lane holds key 8*(r/4) + 4*hh + r%4); the same
    // keys are masked for every head of the wave
    if (k0 + KT - 1 > qpos_lo) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = 8 * (r >> 2) + 4 * hh + (r & 3);
        const bool keep0 = k0 + kr <= qpos;
        const bool keep1 = k0 + 32 + kr <= qpos;
#pragma unroll
        for (int h = 0; h < HW; ++h) {
          c0[h][r] = keep0 ? c0[h][r] : -INFINITY;
          c1[h][r] = keep1 ? c1[h][r] : -INFINITY;
        }
      }
    }
    bool any_grow = false;
    float tmax[HW];
#pragma unroll
    for (int h = 0; h < HW; ++h) {
      float rmax = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) rmax = fmaxf(fmaxf(rmax, c0[h][r]), c1[h][r]);
      tmax[h] = xor32_max(rmax) * sl;  // scale > 0 keeps the order
      any_grow = any_grow || (tmax[h] > m[h] + kRescaleSlack);
    }
    if (__builtin_amdgcn_ballot_w64(any_grow)) {
#pragma unroll
      for (int h = 0; h < HW; ++h) {
        const bool grow = tmax[h] > m[h] + kRescaleSlack;
        const float m_new = grow ? tmax[h] : m[h];
        const float alpha = (m[h] == -INFINITY) ? 0.f : fast_exp2(m[h] - m_new);
        m[h] = m_new;
        l[h] *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[h][dt][r] *= alpha;
      }
    }
    // From here to the P.V products the code is one basic block: the
    // scores of the next tile (independent of this tile's softmax; on the
    // last step the buffer holds the zero-filled tile past the end and the
    // result is not used) are interleaved with the exponentials below, so
    // the matrix and vector units work at the same time.
#if PA_PREFILL_LOOKAHEAD
    f32x16_t n0[HW], n1[HW];
    qk(sk[b1], n0, n1);
#else
    (void)b1;
#endif
    bf16x8_t pb[HW][4];
#pragma unroll
    for (int h = 0; h < HW; ++h) {
      const float nm = (m[h] == -INFINITY) ? 0.f : -m[h];  // rows with no key yet: every score is -inf
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        c0[h][r] = fast_exp2(fmaf(c0[h][r], sl, nm));
        c1[h][r] = fast_exp2(fmaf(c1[h][r], sl, nm));
      }
      // P^T in the B layout: k-step (sub-tile st, half u) = registers
      // 8u..8u+7 of c_st, i.e. keys st*32 + 16u + 8*(e/4) + 4*hh + e%4
      pb[h][0] = pack8(c0[h], 0);
      pb[h][1] = pack8(c0[h], 8);
      pb[h][2] = pack8(c1[h], 0);
      pb[h][3] = pack8(c1[h], 8);
      // the running sum takes the same bf16 weights that multiply V, two
      // at a time (v_dot2_f32_bf16 against ones), so numerator and
      // denominator agree
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint4 w = __builtin_bit_cast(uint4, pb[h][u]);
        ps = dot2_bf16(w.x, kBf16PairOnes, ps);
        ps = dot2_bf16(w.y, kBf16PairOnes, ps);
        ps = dot2_bf16(w.z, kBf16PairOnes, ps);
        ps = dot2_bf16(w.w, kBf16PairOnes, ps);
      }
      l[h] += ps;
    }

    // O^T += V^T P^T; the A operand takes the same keys from row d of V^T,
    // and each V^T fragment read from LDS feeds HW products.  The A operand
    // comes from transposing LDS reads of the row-major V tile: in each
    // 16-lane group, source lane s reads 4 d-values of one key (key K0 +
    // s/4, d = D0 + 4 (s%4)) and lane o receives d = D0 + o of keys K0 ..
    // K0+3; two reads give the 8 keys of the B operand's k-step.  Lane s of
    // 16-lane group g reads, for tile dt and k-step ks, key (ks / 2) 32 +
    // (ks % 2) 16 + 4 (g / 2) + s / 4 (+8 for the second read), slot
    // (2 (g % 2) + (s / 2) % 2) ^ ((key / 4) % 4), half s % 2 (address
    // arithmetic in the LDS address space, constants last, so that they
    // fold into the instructions' offset fields)
    typedef __attribute__((address_space(3))) const char *lds_cptr;
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s *lds_v4s_ptr;
    // the two per-lane bases pass through an empty asm statement: opaque
    // vector values, so that base + constant selects the instructions'
    // offset field instead of a separate address per read
    uint32_t va0 = (uint32_t)(size_t)((lds_cptr)(const char *)sv[b0] + v_off0);
    uint32_t va1 = (uint32_t)(size_t)((lds_cptr)(const char *)sv[b0] + v_off1);
    asm volatile("" : "+v"(va0), "+v"(va1));
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const uint32_t c = dt * 4096 + ((ks >> 1) * 32 + (ks & 1) * 16) * 64;
        const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(size_t)(va0 + c));
        const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_ptr)(size_t)(va1 + c));
        const uint2 l2 = __builtin_bit_cast(uint2, lo);
        const uint2 h2 = __builtin_bit_cast(uint2, hi);
        const bf16x8_t av = as_bf16x8(make_uint4(l2.x, l2.y, h2.x, h2.y));
#pragma unroll
        for (int h = 0; h < HW; ++h) o[h][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[h][ks], o[h][dt], 0, 0, 0);
      }
    }

    if (tid < kMaxTileBlocks) sid[b0][tid] = next_id;  // ids of tile t+3
    __builtin_amdgcn_s_waitcnt(0);  // this wave's loads of tile t+2 are in LDS
    __syncthreads();
#if PA_PREFILL_LOOKAHEAD
#pragma unroll
    for (int h = 0; h < HW; ++h) {
      c0[h] = n0[h];
      c1[h] = n1[h];
    }
#endif
  }

  float lsum[HW];
#pragma unroll
  for (int h = 0; h < HW; ++h) lsum[h] = xor32_sum(l[h]);  // cross-lane: before the divergent store
  if (cascade) {
    // partials (reference max in base-2 units, sum, unnormalised output)
    if (qvalid) {
#pragma unroll
      for (int h = 0; h < HW; ++h) {
        const size_t idx = ((size_t)(r0 + t) * a.num_heads + head0 + h) * a.ws_parts + kchunk;
        float *orow = a.ws_o + idx * DV;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int rq = 0; rq < 4; ++rq) {
            const int d0 = dt * 32 + 8 * rq + 4 * hh;
            *reinterpret_cast<float4 *>(orow + d0) =
                make_float4(o[h][dt][4 * rq], o[h][dt][4 * rq + 1], o[h][dt][4 * rq + 2], o[h][dt][4 * rq + 3]);
          }
        if (hh == 0) {
          a.ws_m[idx] = m[h];
          a.ws_l[idx] = lsum[h];
        }
      }
    }
    return;
  }
  if (qvalid) {
#pragma unroll
    for (int h = 0; h < HW; ++h) {
      const float lt = lsum[h];
      uint16_t *orow = static_cast<uint16_t *>(a.out) + ((size_t)(r0 + t) * a.num_heads + head0 + h) * DV;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const int d0 = dt * 32 + 8 * rq + 4 * hh;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = (lt > 0.f) ? o[h][dt][4 * rq + e] / lt : 0.f;
          *reinterpret_cast<uint2 *>(orow + d0) = make_uint2(pack_bf16x2_rne(v[0], v[1]), pack_bf16x2_rne(v[2], v[3]));
        }
    }
  }
}

template <int D, int DV, int G>
static hipError_t launch_t(const PrefillArgs &a, hipStream_t stream) {
  using Sh = PrefillShape<G>;
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
  k.n_qtiles = (a.max_query_len + Sh::QT - 1) / Sh::QT;
  k.n_chunks = a.group_start ? a.shared_chunks : 1;
  k.chunk = a.shared_chunk;
  const int64_t n_work = (int64_t)a.num_seqs * a.cache.num_kv_heads * Sh::HALVES * k.n_qtiles * k.n_chunks;
  if (n_work <= 0) return hipSuccess;
  if (n_work > (int64_t)0x7fffffff - 8) return hipErrorInvalidConfiguration;
  k.n_work = (int)n_work;
  k.scale_log2 = a.scale * kLog2e;
  k.group_start = a.group_start;
  k.shared_len = a.shared_len;
  k.ws_m = a.ws_m;
  k.ws_l = a.ws_l;
  k.ws_o = a.ws_o;
  k.ws_parts = a.ws_parts;
  const unsigned grid = (unsigned)((n_work + 7) / 8 * 8);
  hipLaunchKernelGGL((prefill_chunk_kernel<D, DV, G>), dim3(grid), dim3(kPrefillThreads), 0, stream, k);
  return hipGetLastError();
}

template <int D, int DV>
static hipError_t launch_g(const PrefillArgs &a, hipStream_t stream) {
  switch (a.num_heads / a.cache.num_kv_heads) {
    case 1: return launch_t<D, DV, 1>(a, stream);
    case 2: return launch_t<D, DV, 2>(a, stream);
    case 4: return launch_t<D, DV, 4>(a, stream);
    case 8: return launch_t<D, DV, 8>(a, stream);
  }
  return hipErrorNotSupported;
}

hipError_t launch_prefill_chunk(const PrefillArgs &a, hipStream_t stream) {
  if (a.cache.dtype != 1) return hipErrorNotSupported;
  const int dk = a.cache.head_dim, dv = a.cache.head_dim_v;
  if (dk == 64 && dv == 64) return launch_g<64, 64>(a, stream);
  if (dk == 128 && dv == 128) return launch_g<128, 128>(a, stream);
  if (dk == 128 && dv == 64) return launch_g<128, 64>(a, stream);
  if (dk == 64 && dv == 128) return launch_g<64, 128>(a, stream);
  return hipErrorNotSupported;
}

}  // namespace pa
