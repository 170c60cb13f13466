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
//  * LDS holds three K and three V tiles.  In step t a wave computes the
//    scores of tile t+1 while it runs the softmax of tile t (independent
//    work for the matrix and vector units), then multiplies V of tile t;
//    the global loads of tile t+2 are in flight meanwhile and are stored
//    before the step's single barrier.
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

// Gather of one K/V tile (keys k0 .. k0+63) from the pool into registers.
// The tile's block ids come from a small LDS array filled ahead of time, so
// no load waits on a block-table read.  Each lane's loads have fixed
// (key, column) slots:
//   K: chunk i = tid + 512 j is key i / C16, 16-byte column i % C16 (whole
//      rows coalesced);
//   V: a lane takes keys 2p, 2p+1 (same block) of one column chunk so that
//      it can write (V[2p][d], V[2p+1][d]) dword pairs of the transposed tile.
// Loads are unconditional: a key at or past kend, or in an invalid block,
// reads the first row of the pool instead and is zeroed when stored.
// waves per work-group (8: one work-group per CU shares each tile among
// 8 waves; 4: two work-groups per CU, whose phases drift apart)
#ifndef PA_PREFILL_INTERLEAVE
#define PA_PREFILL_INTERLEAVE 0
#endif
#ifndef PA_PREFILL_WAVES
#define PA_PREFILL_WAVES 8
#endif
constexpr int kPrefillThreads = 64 * PA_PREFILL_WAVES;
#ifndef PA_PREFILL_VPAD
#define PA_PREFILL_VPAD 4
#endif
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

template <int D, int DV>
struct TileRegs {
  static constexpr int C16K = D / 8;   // 16-byte chunks of a K row
  static constexpr int C16V = DV / 8;  // of a V row
  static constexpr int NK = (64 * C16K + kPrefillThreads - 1) / kPrefillThreads;  // K chunks per thread
  static constexpr int NV = (32 * C16V + kPrefillThreads - 1) / kPrefillThreads;  // V key pairs per thread
  uint4 k[NK];
  uint4 va[NV], vb[NV];
  bool kok[NK], vaok[NV], vbok[NV];
};

// Per-thread constants of the tile gather.  A tile starts at a multiple of
// 64 keys and the block size divides 64, so a thread's key, its block's
// index inside the tile, its row inside that block and its 16-byte column
// are the same for every tile; only the block ids change.
template <int D, int DV>
struct TileLanes {
  using R = TileRegs<D, DV>;
  int kkey[R::NK];   // key of K chunk j (or 64: no chunk)
  int kblk[R::NK];   // its block's index inside the tile
  uint32_t koff[R::NK];  // element offset inside the block
  int vkey[R::NV];   // first key of V pair j (or 64)
  int vblk[R::NV];
  uint32_t voff[R::NV];
};

constexpr int kMaxTileBlocks = 8;  // 64 keys / smallest block size

template <int D, int DV>
__device__ __forceinline__ void tile_lanes(TileLanes<D, DV> &t, int tid, int shift, int bs_mask,
                                           uint32_t k_slot_stride, uint32_t v_slot_stride) {
  using R = TileRegs<D, DV>;
#pragma unroll
  for (int j = 0; j < R::NK; ++j) {
    const int i = tid + kPrefillThreads * j;
    const int key = (i < 64 * R::C16K) ? (i / R::C16K) : 64;
    t.kkey[j] = key;
    t.kblk[j] = (key & 63) >> shift;
    t.koff[j] = (uint32_t)(key & bs_mask) * k_slot_stride + (uint32_t)(i % R::C16K) * 8;
  }
#pragma unroll
  for (int j = 0; j < R::NV; ++j) {
    const int i = tid + kPrefillThreads * j;
    const int key = (i < 32 * R::C16V) ? 2 * (i % 32) : 64;
    t.vkey[j] = key;
    t.vblk[j] = (key & 63) >> shift;
    t.voff[j] = (uint32_t)(key & bs_mask) * v_slot_stride + (uint32_t)((i / 32) % R::C16V) * 8;
  }
}

// block ids of the tile starting at key k0 (64 / block_size entries); the
// work-group keeps them in a tiny LDS array, filled ahead of time
__device__ __forceinline__ int tile_block_id(const int32_t *bt, int k0, int j, int shift, int max_blocks) {
  return bt[min((k0 >> shift) + j, max_blocks - 1)];
}

// Gather of one K/V tile (keys k0 .. k0+63) into registers.  Loads are
// unconditional: a key at or past kend, or in an invalid block, reads a row
// of block 0 instead (inside the pool) and is fixed when stored.
template <int D, int DV>
__device__ __forceinline__ void tile_load(TileRegs<D, DV> &r, const TileLanes<D, DV> &t, const int *ids,
                                          const uint16_t *kbase, const uint16_t *vbase, int k0, int kend,
                                          int num_blocks, size_t k_block_stride, size_t v_block_stride,
                                          uint32_t v_slot_stride) {
  using R = TileRegs<D, DV>;
#pragma unroll
  for (int j = 0; j < R::NK; ++j) {
    const int blk = ids[t.kblk[j]];
    const bool ok = (t.kkey[j] < 64) && ((unsigned)blk < (unsigned)num_blocks);
    const size_t base = (size_t)(ok ? blk : 0) * k_block_stride + t.koff[j];
    r.k[j] = *reinterpret_cast<const uint4 *>(kbase + base);
    r.kok[j] = ok || t.kkey[j] >= 64;  // K of a masked key needs no fix: its score is replaced
  }
#pragma unroll
  for (int j = 0; j < R::NV; ++j) {
    const int blk = ids[t.vblk[j]];  // keys 2p and 2p+1 share a block
    const bool inb = (t.vkey[j] < 64) && ((unsigned)blk < (unsigned)num_blocks);
    const size_t base = (size_t)(inb ? blk : 0) * v_block_stride + t.voff[j];
    r.va[j] = *reinterpret_cast<const uint4 *>(vbase + base);
    r.vb[j] = *reinterpret_cast<const uint4 *>(vbase + base + v_slot_stride);
    r.vaok[j] = inb && (k0 + t.vkey[j] < kend);
    r.vbok[j] = inb && (k0 + t.vkey[j] + 1 < kend);
  }
}

// component-wise (a ?: 0); a select on the vector objects themselves would
// pick between their addresses and force both into scratch memory
__device__ __forceinline__ uint4 keep_if(bool ok, const uint4 &v) {
  return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
}

template <int D, int DV, int KSTR, int VSTR>
__device__ __forceinline__ void tile_store(TileRegs<D, DV> &r, uint16_t *sk, uint16_t *svt, int tid) {
  using R = TileRegs<D, DV>;
  // zero what must not enter the products (rare: the last tile, or a block
  // id outside the pool); the common full tile skips the selects
  bool all_ok = true;
#pragma unroll
  for (int j = 0; j < R::NK; ++j) all_ok = all_ok && r.kok[j];
#pragma unroll
  for (int j = 0; j < R::NV; ++j) all_ok = all_ok && r.vaok[j] && r.vbok[j];
  if (!all_ok) {
#pragma unroll
    for (int j = 0; j < R::NK; ++j) r.k[j] = keep_if(r.kok[j], r.k[j]);
#pragma unroll
    for (int j = 0; j < R::NV; ++j) {
      r.va[j] = keep_if(r.vaok[j], r.va[j]);
      r.vb[j] = keep_if(r.vbok[j], r.vb[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < R::NK; ++j) {
    const int i = tid + kPrefillThreads * j;
    if (i < 64 * R::C16K) *reinterpret_cast<uint4 *>(sk + (i / R::C16K) * KSTR + (i % R::C16K) * 8) = r.k[j];
  }
#pragma unroll
  for (int j = 0; j < R::NV; ++j) {
    const int i = tid + kPrefillThreads * j;
    if (i < 32 * R::C16V) {
      const int p = i % 32;
      const int c = i / 32;
      uint32_t *dst = reinterpret_cast<uint32_t *>(svt + (c * 8) * VSTR + 2 * p);
      constexpr int W = VSTR / 2;  // dwords per V^T row
      const uint4 a = r.va[j];
      const uint4 b = r.vb[j];
      dst[0 * W] = interleave_lo(a.x, b.x);
      dst[1 * W] = interleave_hi(a.x, b.x);
      dst[2 * W] = interleave_lo(a.y, b.y);
      dst[3 * W] = interleave_hi(a.y, b.y);
      dst[4 * W] = interleave_lo(a.z, b.z);
      dst[5 * W] = interleave_hi(a.z, b.z);
      dst[6 * W] = interleave_lo(a.w, b.w);
      dst[7 * W] = interleave_hi(a.w, b.w);
    }
  }
}

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
  constexpr int KSTR = D + 8;        // LDS row stride of K, bf16 elements
  constexpr int VSTR = KT + PA_PREFILL_VPAD;  // LDS row stride of V^T, bf16 elements
  constexpr int NDS = D / 16;        // k-steps of Q K^T
  constexpr int NDT = DV / 32;       // 32-row tiles of O^T

  // three buffers each for K and V: at step t the waves read K of tile t+1
  // and V of tile t while tile t+2 is stored
  __shared__ __attribute__((aligned(16))) uint16_t sk[3][KT * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t svt[3][DV * VSTR];
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
  TileLanes<D, DV> lanes;
  tile_lanes<D, DV>(lanes, tid, shift, bs_mask, slot_stride, vslot_stride);

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
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t *>(skb + col * KSTR + ds * 16 + hh * 8);
      const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t *>(skb + (32 + col) * KSTR + ds * 16 + hh * 8);
#pragma unroll
      for (int h = 0; h < HW; ++h) {
        s0[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qb[h][ds], s0[h], 0, 0, 0);
        s1[h] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qb[h][ds], s1[h], 0, 0, 0);
      }
    }
  };

  // Pipeline, one barrier per step t:
  //   loads of tile t+2 -> registers;  S(t+1) = K(t+1) Q^T;  softmax of S(t);
  //   O += V(t) P(t);  registers -> LDS buffers of tile t+2.
  // Block ids: sid[j % 3] holds the ids of tile j, filled three tiles ahead.
  if (tid < kMaxTileBlocks) {
#pragma unroll
    for (int j = 0; j < 3; ++j) sid[j][tid] = tile_block_id(bt, kbeg + j * KT, tid, shift, a.max_blocks_per_seq);
  }
  __syncthreads();
  TileRegs<D, DV> tr;
  const int ntiles = (kend - kbeg + KT - 1) / KT;
  tile_load<D, DV>(tr, lanes, sid[0], kbase, vbase, kbeg, kend, a.num_blocks, block_stride, vblock_stride,
                   vslot_stride);
  tile_store<D, DV, KSTR, VSTR>(tr, sk[0], svt[0], tid);
  tile_load<D, DV>(tr, lanes, sid[1], kbase, vbase, kbeg + KT, kend, a.num_blocks, block_stride, vblock_stride,
                   vslot_stride);
  tile_store<D, DV, KSTR, VSTR>(tr, sk[1], svt[1], tid);
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
    // tile t+2 from the pool (past the last tile: in-pool rows, zeroed)
    tile_load<D, DV>(tr, lanes, sid[b2], kbase, vbase, k0 + 2 * KT, kend, a.num_blocks, block_stride,
                     vblock_stride, vslot_stride);
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
    // and each V^T fragment read from LDS feeds HW products
    const uint16_t *svb = svt[b0];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const uint16_t *vrow = svb + (dt * 32 + col) * VSTR;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int kb0 = (ks >> 1) * 32 + (ks & 1) * 16 + 4 * hh;
        const uint2 lo = *reinterpret_cast<const uint2 *>(vrow + kb0);
        const uint2 hi = *reinterpret_cast<const uint2 *>(vrow + kb0 + 8);
        const bf16x8_t av = as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
        for (int h = 0; h < HW; ++h) o[h][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[h][ks], o[h][dt], 0, 0, 0);
      }
    }

    tile_store<D, DV, KSTR, VSTR>(tr, sk[b2], svt[b2], tid);
    if (tid < kMaxTileBlocks) sid[b0][tid] = next_id;  // ids of tile t+3
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
