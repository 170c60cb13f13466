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
#ifndef PA_PREFILL_ORDER
#define PA_PREFILL_ORDER 1
#endif

template <int D>
struct TileRegs {
  static constexpr int C16 = D / 8;
  static constexpr int NK = (64 * C16 + kPrefillThreads - 1) / kPrefillThreads;  // K chunks per thread
  static constexpr int NV = (32 * C16 + kPrefillThreads - 1) / kPrefillThreads;  // V key pairs per thread
  uint4 k[NK];
  uint4 va[NV], vb[NV];
  bool kok[NK], vaok[NV], vbok[NV];
};

// Per-thread constants of the tile gather.  A tile starts at a multiple of
// 64 keys and the block size divides 64, so a thread's key, its block's
// index inside the tile, its row inside that block and its 16-byte column
// are the same for every tile; only the block ids change.
template <int D>
struct TileLanes {
  static constexpr int C16 = D / 8;
  int kkey[TileRegs<D>::NK];   // key of K chunk j (or 64: no chunk)
  int kblk[TileRegs<D>::NK];   // its block's index inside the tile
  uint32_t koff[TileRegs<D>::NK];  // element offset inside the block
  int vkey[TileRegs<D>::NV];   // first key of V pair j (or 64)
  int vblk[TileRegs<D>::NV];
  uint32_t voff[TileRegs<D>::NV];
};

constexpr int kMaxTileBlocks = 8;  // 64 keys / smallest block size

template <int D>
__device__ __forceinline__ void tile_lanes(TileLanes<D> &t, int tid, int shift, int bs_mask, uint32_t slot_stride) {
  constexpr int C16 = D / 8;
#pragma unroll
  for (int j = 0; j < TileRegs<D>::NK; ++j) {
    const int i = tid + kPrefillThreads * j;
    const int key = (i < 64 * C16) ? (i / C16) : 64;
    t.kkey[j] = key;
    t.kblk[j] = (key & 63) >> shift;
    t.koff[j] = (uint32_t)(key & bs_mask) * slot_stride + (uint32_t)(i % C16) * 8;
  }
#pragma unroll
  for (int j = 0; j < TileRegs<D>::NV; ++j) {
    const int i = tid + kPrefillThreads * j;
    const int key = (i < 32 * C16) ? 2 * (i % 32) : 64;
    t.vkey[j] = key;
    t.vblk[j] = (key & 63) >> shift;
    t.voff[j] = (uint32_t)(key & bs_mask) * slot_stride + (uint32_t)((i / 32) % C16) * 8;
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
template <int D>
__device__ __forceinline__ void tile_load(TileRegs<D> &r, const TileLanes<D> &t, const int *ids,
                                          const uint16_t *kbase, const uint16_t *vbase, int k0, int kend,
                                          int num_blocks, size_t block_stride, uint32_t slot_stride) {
#pragma unroll
  for (int j = 0; j < TileRegs<D>::NK; ++j) {
    const int blk = ids[t.kblk[j]];
    const bool ok = (t.kkey[j] < 64) && ((unsigned)blk < (unsigned)num_blocks);
    const size_t base = (size_t)(ok ? blk : 0) * block_stride + t.koff[j];
    r.k[j] = *reinterpret_cast<const uint4 *>(kbase + base);
    r.kok[j] = ok || t.kkey[j] >= 64;  // K of a masked key needs no fix: its score is replaced
  }
#pragma unroll
  for (int j = 0; j < TileRegs<D>::NV; ++j) {
    const int blk = ids[t.vblk[j]];  // keys 2p and 2p+1 share a block
    const bool inb = (t.vkey[j] < 64) && ((unsigned)blk < (unsigned)num_blocks);
    const size_t base = (size_t)(inb ? blk : 0) * block_stride + t.voff[j];
    r.va[j] = *reinterpret_cast<const uint4 *>(vbase + base);
    r.vb[j] = *reinterpret_cast<const uint4 *>(vbase + base + slot_stride);
    r.vaok[j] = inb && (k0 + t.vkey[j] < kend);
    r.vbok[j] = inb && (k0 + t.vkey[j] + 1 < kend);
  }
}

// component-wise (a ?: 0); a select on the vector objects themselves would
// pick between their addresses and force both into scratch memory
__device__ __forceinline__ uint4 keep_if(bool ok, const uint4 &v) {
  return make_uint4(ok ? v.x : 0u, ok ? v.y : 0u, ok ? v.z : 0u, ok ? v.w : 0u);
}

template <int D, int KSTR, int VSTR>
__device__ __forceinline__ void tile_store(TileRegs<D> &r, uint16_t *sk, uint16_t *svt, int tid) {
  constexpr int C16 = D / 8;
  // zero what must not enter the products (rare: the last tile, or a block
  // id outside the pool); the common full tile skips the selects
  bool all_ok = true;
#pragma unroll
  for (int j = 0; j < TileRegs<D>::NK; ++j) all_ok = all_ok && r.kok[j];
#pragma unroll
  for (int j = 0; j < TileRegs<D>::NV; ++j) all_ok = all_ok && r.vaok[j] && r.vbok[j];
  if (!all_ok) {
#pragma unroll
    for (int j = 0; j < TileRegs<D>::NK; ++j) r.k[j] = keep_if(r.kok[j], r.k[j]);
#pragma unroll
    for (int j = 0; j < TileRegs<D>::NV; ++j) {
      r.va[j] = keep_if(r.vaok[j], r.va[j]);
      r.vb[j] = keep_if(r.vbok[j], r.vb[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < TileRegs<D>::NK; ++j) {
    const int i = tid + kPrefillThreads * j;
    if (i < 64 * C16) *reinterpret_cast<uint4 *>(sk + (i / C16) * KSTR + (i % C16) * 8) = r.k[j];
  }
#pragma unroll
  for (int j = 0; j < TileRegs<D>::NV; ++j) {
    const int i = tid + kPrefillThreads * j;
    if (i < 32 * C16) {
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

template <int D, int G>
__global__ void __launch_bounds__(kPrefillThreads, 8 / PA_PREFILL_WAVES)
prefill_chunk_kernel(const PrefillKernelArgs a) {
  constexpr int NW = kPrefillThreads / 64;
  constexpr int GW = G < NW ? G : NW;  // query heads per work-group
  constexpr int HALVES = G / GW;       // work-groups per kv head along heads
  constexpr int TG = NW / GW;          // 32-token query groups per work-group
  constexpr int QT = 32 * TG;        // query tokens per work-group
  constexpr int KT = 64;             // keys per tile
  constexpr int KSTR = D + 8;        // LDS row stride of K, bf16 elements
  constexpr int VSTR = KT + PA_PREFILL_VPAD;  // LDS row stride of V^T, bf16 elements
  constexpr int NDS = D / 16;        // k-steps of Q K^T
  constexpr int NDT = D / 32;        // 32-row tiles of O^T

  // three buffers each for K and V: at step t the waves read K of tile t+1
  // and V of tile t while tile t+2 is stored
  __shared__ __attribute__((aligned(16))) uint16_t sk[3][KT * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t svt[3][D * VSTR];
  __shared__ int sid[3][kMaxTileBlocks];

  // Work id.  Work-groups are dispatched round-robin over the 8 XCDs; the
  // remap gives each XCD a contiguous range of work ids.  Ids are ordered
  // (kv head, head half, query tile from the last, sequence), so an XCD
  // serves whole kv heads of every sequence (equal work per XCD when the
  // head groups are a multiple of 8), all query tiles of a (sequence, kv
  // head) share one L2, and the tiles with the most keys start first.
  const int nwg = gridDim.x;  // a multiple of 8
  const int bid = blockIdx.x;
  const int wid = (bid & 7) * (nwg >> 3) + (bid >> 3);
  if (wid >= a.n_work) return;
  int rest = wid;
#if PA_PREFILL_ORDER == 1
  const int qt_rev = rest % a.n_qtiles;
  rest /= a.n_qtiles;
  const int seq = rest % a.num_seqs;
  rest /= a.num_seqs;
#else
  const int seq = rest % a.num_seqs;
  rest /= a.num_seqs;
  const int qt_rev = rest % a.n_qtiles;
  rest /= a.n_qtiles;
#endif
  const int half = rest % HALVES;
  const int kvh = rest / HALVES;
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

  const uint32_t slot_stride = (uint32_t)a.num_kv_heads * D;
  const size_t block_stride = (size_t)slot_stride << a.block_shift;
  const uint16_t *kbase = static_cast<const uint16_t *>(a.k_cache) + (size_t)kvh * D;
  const uint16_t *vbase = static_cast<const uint16_t *>(a.v_cache) + (size_t)kvh * D;
  const int32_t *bt = a.block_tables + (size_t)seq * a.max_blocks_per_seq;
  const int shift = a.block_shift;
  const int bs_mask = (1 << shift) - 1;
  const float sl = a.scale_log2;
  TileLanes<D> lanes;
  tile_lanes<D>(lanes, tid, shift, bs_mask, slot_stride);

  float m = -INFINITY;  // reference max of this lane's query (base-2 units)
  float l = 0.f;        // running sum over this lane's keys
  f32x16_t o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;

  // S^T tile of keys k0 .. k0+63 (s0: first 32 keys, s1: last 32)
  auto qk = [&](const uint16_t *skb, f32x16_t &s0, f32x16_t &s1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = 0.f;
      s1[r] = 0.f;
    }
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t *>(skb + col * KSTR + ds * 16 + hh * 8);
      const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t *>(skb + (32 + col) * KSTR + ds * 16 + hh * 8);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qb[ds], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qb[ds], s1, 0, 0, 0);
    }
  };

  // Pipeline, one barrier per step t:
  //   loads of tile t+2 -> registers;  S(t+1) = K(t+1) Q^T;  softmax of S(t);
  //   O += V(t) P(t);  registers -> LDS buffers of tile t+2.
  // Block ids: sid[j % 3] holds the ids of tile j, filled three tiles ahead.
  if (tid < kMaxTileBlocks) {
#pragma unroll
    for (int j = 0; j < 3; ++j) sid[j][tid] = tile_block_id(bt, j * KT, tid, shift, a.max_blocks_per_seq);
  }
  __syncthreads();
  TileRegs<D> tr;
  tile_load<D>(tr, lanes, sid[0], kbase, vbase, 0, kend, a.num_blocks, block_stride, slot_stride);
  tile_store<D, KSTR, VSTR>(tr, sk[0], svt[0], tid);
  tile_load<D>(tr, lanes, sid[1], kbase, vbase, KT, kend, a.num_blocks, block_stride, slot_stride);
  tile_store<D, KSTR, VSTR>(tr, sk[1], svt[1], tid);
  __syncthreads();

  f32x16_t c0, c1;  // S of the current tile
  qk(sk[0], c0, c1);

  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * KT;
    const int b0 = kt % 3;
    const int b1 = (kt + 1) % 3;
    const int b2 = (kt + 2) % 3;
    // tile t+2 from the pool (past the last tile: in-pool rows, zeroed)
    tile_load<D>(tr, lanes, sid[b2], kbase, vbase, k0 + 2 * KT, kend, a.num_blocks, block_stride, slot_stride);
    int next_id = 0;
    if (tid < kMaxTileBlocks) next_id = tile_block_id(bt, k0 + 3 * KT, tid, shift, a.max_blocks_per_seq);

    // causal mask on tiles that cross this wave's diagonal (raw scores;
    // register r of this lane holds key 8*(r/4) + 4*hh + r%4)
    if (k0 + KT - 1 > prefix + tw0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = 8 * (r >> 2) + 4 * hh + (r & 3);
        c0[r] = (k0 + kr <= qpos) ? c0[r] : -INFINITY;
        c1[r] = (k0 + 32 + kr <= qpos) ? c1[r] : -INFINITY;
      }
    }
    float rmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) rmax = fmaxf(fmaxf(rmax, c0[r]), c1[r]);
    const float tmax = xor32_max(rmax) * sl;  // scale > 0 keeps the order
    const bool grow = tmax > m + kRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? tmax : m;
      const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - m_new);
      m = m_new;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    }
    // From here to the P.V products the code is one basic block: the
    // scores of the next tile (independent of this tile's softmax; on the
    // last step the buffer holds the zero-filled tile past the end and the
    // result is not used) are interleaved with the exponentials below, so
    // the matrix and vector units work at the same time.
    f32x16_t n0, n1;
    qk(sk[b1], n0, n1);
    const float nm = (m == -INFINITY) ? 0.f : -m;  // rows with no key yet: every score is -inf
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      c0[r] = fast_exp2(fmaf(c0[r], sl, nm));
      c1[r] = fast_exp2(fmaf(c1[r], sl, nm));
    }
#if PA_PREFILL_INTERLEAVE
#pragma unroll
    for (int i = 0; i < 2 * NDS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, PA_PREFILL_INTERLEAVE, 0);  // some VALU
    }
#endif

    // P^T in the B layout: k-step (sub-tile st, half u) = registers 8u..8u+7
    // of c_st, i.e. keys st*32 + 16u + 8*(e/4) + 4*hh + e%4 for slot e
    bf16x8_t pb[4];
    pb[0] = pack8(c0, 0);
    pb[1] = pack8(c0, 8);
    pb[2] = pack8(c1, 0);
    pb[3] = pack8(c1, 8);
    // the running sum takes the same bf16 weights that multiply V, two at a
    // time (v_dot2_f32_bf16 against ones), so numerator and denominator agree
    {
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint4 w = __builtin_bit_cast(uint4, pb[u]);
        ps = dot2_bf16(w.x, kBf16PairOnes, ps);
        ps = dot2_bf16(w.y, kBf16PairOnes, ps);
        ps = dot2_bf16(w.z, kBf16PairOnes, ps);
        ps = dot2_bf16(w.w, kBf16PairOnes, ps);
      }
      l += ps;
    }

    // O^T += V^T P^T; the A operand takes the same keys from row d of V^T
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
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[ks], o[dt], 0, 0, 0);
      }
    }

    tile_store<D, KSTR, VSTR>(tr, sk[b2], svt[b2], tid);
    if (tid < kMaxTileBlocks) sid[b0][tid] = next_id;  // ids of tile t+3
    __syncthreads();
    c0 = n0;
    c1 = n1;
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
  constexpr int NW = kPrefillThreads / 64;
  constexpr int GW = G < NW ? G : NW;
  constexpr int HALVES = G / GW;
  constexpr int QT = 32 * (NW / GW);
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
  hipLaunchKernelGGL((prefill_chunk_kernel<D, G>), dim3(grid), dim3(kPrefillThreads), 0, stream, k);
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
