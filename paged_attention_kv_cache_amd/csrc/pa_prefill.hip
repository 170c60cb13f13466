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
//  * A work-group (4 waves, two per CU) serves one kv head: 4 of its
//    query heads x 32 tokens of one sequence's chunk (fewer heads and more
//    32-token groups for G < 4; G = 8 takes two work-groups).  Every K/V
//    tile is gathered once per work-group and shared by its waves through
//    LDS.  Small work items (32 queries at G = 4) let the CUs share a
//    launch evenly, and the two work-groups of a CU, which do not wait for
//    each other, fill each other's stalls.
//  * K/V tiles of 64 keys are gathered through the block table straight
//    into LDS with 16-byte global-to-LDS loads (no registers, no LDS store
//    instructions), both row-major [key][d] in swizzled 64-byte chunk
//    groups (see TileGather).  A wave's loads of a tile cover 16 keys,
//    which lie in one block for block sizes 16 and 32, so the block id is
//    one scalar load and the block's address a scalar sum.  Keys past the last position
//    the work-group needs, and keys in an invalid block, read a zero chunk
//    instead, so a masked key never brings a NaN into the products.
//  * The scale (times log2(e), so that the softmax uses exp2) multiplies
//    the fp32 scores: each weight is one FMA (score * scale - max) and one
//    exp2.  A negative scale is applied as |scale| to -Q (exact in bf16),
//    which keeps the order of the scaled scores that of the raw ones.
//  * Scores are computed transposed, S^T = K Q^T, on
//    v_mfma_f32_32x32x16_bf16 (A = K from LDS, B = Q^T held in registers).
//    In the accumulator layout every lane then holds 16 keys of one query,
//    so the online-softmax max and sum need one cross-half exchange only,
//    and the rescale factor is a per-lane scalar.
//  * The weights, rounded to bf16, are already in the B-operand layout of
//    O^T += V^T P^T, so P never goes through LDS; the A operand (V^T) comes
//    from the row-major V tile through gfx950's transposing LDS reads.
//  * Online softmax with a lazy reference max: the first tile of a
//    work-group and the tiles that cross the causal diagonal take the max
//    of their scores (and move the reference when it grows by more than
//    2^8).  The tiles in between take no max at all: their weights are
//    exponentials relative to the reference, and only if a lane's sum of
//    them exceeds 2^32 (a score far above the reference) is the tile
//    recomputed with a new reference.  The final division by the running
//    sum makes any reference exact up to rounding.
//  * LDS holds three K and two V tiles.  In step t a wave computes the
//    scores of tile t+1 while it runs the exponentials of tile t
//    (independent work for the matrix and vector units), then multiplies V
//    of tile t; K of tile t+2 and V of tile t+1 are loaded into LDS
//    meanwhile and waited for before the step's single barrier.
//  * Work ids are remapped so that each XCD serves whole kv heads of every
//    sequence: the XCDs get equal work, and the query tiles of one
//    (sequence, kv head), which read the same K/V, share that XCD's L2.
//    Within a kv head the (sequence, query tile) items are dispatched
//    longest first (most key tiles to read), each work-group finding its
//    item from the context lengths (pick_item).
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
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ bf16x8_t pack8(const f32x16_t &s, int base) {
  bf16x8_t r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)s[base + e];
  return r;
}

constexpr int kPrefillWaves = 4;  // waves per work-group, two work-groups per CU (2 waves per SIMD)
constexpr int kPrefillThreads = 64 * kPrefillWaves;
constexpr int KT = 64;            // keys per tile
constexpr int kKBufs = 3;         // K tiles in LDS: scores of t+1 read, t+2 loading, t kept
constexpr int kVBufs = 2;         // V tiles in LDS: P.V of t read, t+1 loading

typedef const __attribute__((address_space(4))) int32_t *tab_ptr_t;  // scalar loads of table entries
typedef __attribute__((address_space(3))) void *lds_ptr_t;

// source of the 16-byte chunks of keys that must read as zero (blocks of 8;
// a wave's loads of one tile read it at offsets of up to 192 bytes)
__device__ const uint4 kZeroChunk[16] = {};
// last word of a raw buffer descriptor (32-bit data format, no swizzle)
constexpr int kRsrcWord3 = 0x00020000;

// The tile loads are issued as inline assembly.  The compiler then does
// not know that they write LDS, so it does not wait for them before the
// step's own LDS reads (of other tiles); the kernel waits for them itself,
// at the end of the step that issues them, before the barrier that precedes
// their first reader.
//
// 16 bytes per lane from a raw buffer of `bytes` bytes at `base` (uniform)
// into LDS at lds_addr + 16 * lane; a lane whose offset is out of range gets
// zeros.  M0 holds the LDS address of the load (one wait state after its
// write).
__device__ __forceinline__ void dma_buffer16(uint32_t lds_addr, uint32_t voffset, const char *base, int bytes) {
  typedef int v4i __attribute__((ext_vector_type(4)));
  const uint64_t b = (uint64_t)base;
  const v4i r = {(int)(uint32_t)b, (int)((uint32_t)(b >> 32) & 0xffffu), bytes, kRsrcWord3};
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voffset), "s"(r)
               : "memory", "m0");
}
// 16 bytes per lane from src into LDS at lds_addr + 16 * lane
__device__ __forceinline__ void dma_global16(uint32_t lds_addr, const void *src) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds_addr), "v"(src)
               : "memory", "m0");
}
// entries i[0..1] of a table row, read through the scalar
// cache and waited for at once (a few cycles from the scalar cache; issued
// where the wave has no LDS reads in flight, so the wait holds up nothing
// else).  The outputs are early-clobber: a load may land before the next
// one has read its inputs.
__device__ __forceinline__ void table_entries2(const int32_t *row, const int (&i)[4], int (&v)[4]) {
  asm volatile("s_load_dword %0, %2, %3\n\ts_load_dword %1, %2, %4\n\ts_waitcnt lgkmcnt(0)"
               : "=&s"(v[0]), "=&s"(v[1])
               : "s"(row), "s"(i[0] * 4), "s"(i[1] * 4)
               : "memory");
  v[2] = v[0];
  v[3] = v[1];
}
// s_waitcnt with only vmcnt = n (n < 64) counted
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Gather of one K (or V) tile, keys k0 .. k0+63 of row width DIM, straight
// from the pool into LDS with 16-byte global-to-LDS loads: no registers, no
// LDS store instructions.  LDS layout: the row's 16-byte chunks in groups of
// four (64 bytes, 32 elements): group g of every key forms a 4 KB block
// [key][4 chunks], and inside a key's 64 bytes chunk c sits in slot
// (c % 4) ^ ((k / 4) % 4).  Sixteen consecutive keys then cover all LDS
// banks for any fixed chunk, and the slot pattern depends on a lane's key
// only through (k / 4) % 4, so every fragment read is a per-lane base plus
// a compile-time offset.  One load writes 1 KB of consecutive LDS (lane i
// at 16 i): 16 keys x one chunk group, each lane fetching the global chunk
// that belongs in its slot.  The NWL waves that share a tile split its
// loads so that all loads of one wave cover the same 16 keys (key group
// wave % 4) and differ only in the chunk group: one block id per wave and
// tile (two with blocks of 8 keys, one per half-wave), and a lane's byte
// offset inside its block that changes by 64 bytes per chunk group.  A tile
// starts at a multiple of 64 keys and the block size divides 64, so that
// offset is the same for every tile; only the block ids change.
struct TileIds {
  int id[2];
};

template <int DIM, int NWL>
struct TileGather {
  static constexpr int CG = DIM / 32;            // chunk groups per row
  static constexpr int PER_WAVE = (CG * 4) / NWL;  // loads per wave and tile
  static constexpr uint32_t kChunkStep = (NWL / 4) * 64;  // bytes between a wave's loads in the block
  static_assert(NWL % 4 == 0 && PER_WAVE >= 1 && (CG * 4) % NWL == 0, "tile split over the waves");
  int kg;          // first key of the wave's 16 keys (wave-uniform)
  uint32_t off0;   // byte offset of this lane's first chunk inside its block
  uint32_t lds0;   // byte offset of the wave's first load inside the tile (wave-uniform)
  int lkey;        // this lane's key within the 16: lane / 4

  __device__ __forceinline__ void init(int wl, int lane, int bs_mask, uint32_t slot_stride) {
    lkey = lane >> 2;
    kg = (wl % 4) * 16;
    const int key = kg + lkey;
    // load j of this wave is tile load j * NWL + wl: key group wl % 4, chunk
    // group j * NWL / 4 + wl / 4
    const int chunk = (wl / 4) * 4 + ((lane % 4) ^ ((key >> 2) & 3));
    off0 = ((uint32_t)(key & bs_mask) * slot_stride + (uint32_t)chunk * 8) * 2u;
    lds0 = (uint32_t)wl * 1024;
  }
  // block ids (wave-uniform) of the wave's 16 keys in the tile at k0, read
  // from the table row (indices clamped into it): id[0], and with blocks of
  // 8 keys id[1] for the upper half-wave
  using Ids = TileIds;
  __device__ __forceinline__ Ids ids(bool kBs8, const int32_t *row, int k0, int shift, int max_blocks) const {
    int idx[4], v[4];
    const int e = (k0 + kg) >> shift;
    idx[0] = __builtin_amdgcn_readfirstlane(min(e, max_blocks - 1));
    idx[1] = __builtin_amdgcn_readfirstlane(min(e + (kBs8 ? 1 : 0), max_blocks - 1));
    table_entries2(row, idx, v);
    Ids r;
    r.id[0] = v[0];
    r.id[1] = v[1];
    return r;
  }
  // the wave's loads of one tile into the LDS tile at lds_tile.  kBs8:
  // blocks of 8 keys; kPartial: keys at or past kend read zeros (the last
  // tiles of a range).  Both are constants at every call.
  __device__ __forceinline__ void issue(bool kBs8, bool kPartial, uint32_t lds_tile, const Ids &ids, const char *base,
                                        const char *zero, int num_blocks, uint32_t block_bytes, int k0, int kend,
                                        int lane) const {
    const bool kok = !kPartial || (k0 + kg + lkey < kend);
    if (!kBs8) {
      // one block for the wave: a buffer over it, empty for an id outside
      // the pool; out-of-range reads (an empty buffer, or a key past kend
      // sent past the end) return zeros
      const int b = ids.id[0];
      const bool bok = (unsigned)b < (unsigned)num_blocks;
      const char *blk = base + (size_t)(unsigned)(bok ? b : 0) * block_bytes;
      const uint32_t vo = kok ? off0 : 0x80000000u;
      const int nbytes = bok ? (int)block_bytes : 0;
#pragma unroll
      for (int j = 0; j < PER_WAVE; ++j)
        dma_buffer16(lds_tile + lds0 + (uint32_t)j * NWL * 1024, vo + (uint32_t)j * kChunkStep, blk, nbytes);
    } else {
      const int b = (lane < 32) ? ids.id[0] : ids.id[1];
      const bool ok = kok && (unsigned)b < (unsigned)num_blocks;
      const char *src = ok ? base + (size_t)(unsigned)b * block_bytes + off0 : zero;
#pragma unroll
      for (int j = 0; j < PER_WAVE; ++j) dma_global16(lds_tile + lds0 + (uint32_t)j * NWL * 1024, src + j * kChunkStep);
    }
  }
};

// the reference max moves on a max-taking tile only when a score exceeds it
// by more than this many base-2 units
constexpr float kRescaleSlack = 8.f;
// a tile without a max is redone when one of a lane's sums of weights
// relative to the reference exceeds this (weights below 2^32 keep the fp32
// sums and bf16 weights far from overflow)
constexpr float kSumLimit = 4294967296.f;

constexpr uint32_t kBf16PairOnes = 0x3F803F80u;  // two bf16 1.0

// Work-group shape for G query heads per kv head: 4 waves, each one query
// head x 32 queries; with G < 4 the waves take more query groups of the
// same heads, with G = 8 a kv head's heads take two work-groups.
template <int G>
struct PrefillShape {
  static constexpr int NW = kPrefillWaves;         // waves per work-group
  static constexpr int GWH = G < NW ? G : NW;      // head slots per work-group
  static constexpr int HALVES = G / GWH;           // work-groups per kv head along heads
  static constexpr int TG = NW / GWH;              // 32-token query groups per work-group
  static constexpr int QT = 32 * TG;               // query tokens per work-group
  static_assert(G % GWH == 0 && NW % GWH == 0, "heads and waves must divide");
};

// sum over the wave of x (0 <= x < 2^bits, bits wave-uniform): one ballot
// and one popcount per bit, all scalar after the compare
__device__ __forceinline__ int wave_sum_bits(int x, int bits) {
  int s = 0;
  for (int b = 0; b < bits; ++b) s += (int)__builtin_popcountll(__builtin_amdgcn_ballot_w64((x >> b) & 1)) << b;
  return s;
}
// the same sum over the lanes below this one
__device__ __forceinline__ int wave_prefix_bits(int x, int bits) {
  int s = 0;
  for (int b = 0; b < bits; ++b) {
    const unsigned long long m = __builtin_amdgcn_ballot_w64((x >> b) & 1);
    s += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u)) << b;
  }
  return s;
}

// sequences up to which a work-group picks its item by size
constexpr int kRankSeqChunks = 4;

// Dispatch order by size.  The items of one (kv head, head part) are the
// pairs (sequence s, query tile qt) with qt * QT < q_len(s); an item reads
// keys = min(context, prefix + QT (qt + 1)) keys.  Its cost class is
// ceil(keys / U) with U = 512 keys (8 key tiles): coarse enough that the
// items of one sequence, which read the same K/V, mostly share a class and
// are dispatched together (their tiles then come into the XCD's L2 about
// once), fine enough to keep the longest first.  The class does not
// decrease with qt, so the number of items of s whose class is at least W
// has a closed form: every qt from (U (W - 1) - prefix) / QT on, if the
// context has more than U (W - 1) keys.  The work-group at dispatch
// position pos takes the pos-th item in (class descending, s ascending, qt
// descending) order: a binary search over W for the class of that item,
// each probe summing the per-sequence counts over the wave (lane =
// sequence, up to 4 per lane), then its rank among the items of that
// class.  Returns false for a position past the last item.  Every wave
// computes the same result from the same values.
template <int QT>
__device__ __forceinline__ bool pick_item(const PrefillKernelArgs &a, int pos, int lane, int &seq_out,
                                          int &qt_out) {
  constexpr int U = 8 * KT;  // keys per cost class
  const int nchunks = (a.num_seqs + 63) / 64;
  int nq[kRankSeqChunks], cx[kRankSeqChunks], pf[kRankSeqChunks];
#pragma unroll
  for (int c = 0; c < kRankSeqChunks; ++c) {
    nq[c] = 0;
    cx[c] = 0;
    pf[c] = 0;
    const int s = c * 64 + lane;
    if (c < nchunks && s < a.num_seqs) {
      const int e1 = min(a.query_start_loc[s + 1], a.num_query_tokens);
      const int e0 = max(0, min(a.query_start_loc[s], e1));
      const int ql = e1 - e0;
      cx[c] = max(0, min(a.context_lens[s], a.ctx_cap));
      pf[c] = cx[c] - ql;
      nq[c] = min((ql + QT - 1) / QT, a.n_qtiles);
    }
  }
  // items of lane's sequences whose class is at least W (all for W <= 0)
  // (64-bit key counts: a context bound near 2^31 keys must not wrap)
  auto above = [&](int W, int c) -> int {
    if (W <= 0) return nq[c];
    const long long kth = (long long)U * (W - 1);
    if (cx[c] <= kth) return 0;
    const long long d = kth - pf[c];
    return max(0, nq[c] - (d > 0 ? (int)(d / QT) : 0));
  };
  const int bits = 34 - __builtin_clz((unsigned)a.n_qtiles);  // 4 chunks of counts < 2 n_qtiles + 1
  auto count_above = [&](int W) -> int {
    int x = 0;
#pragma unroll
    for (int c = 0; c < kRankSeqChunks; ++c) x += above(W, c);
    return wave_sum_bits(x, bits);
  };
  if (pos >= count_above(0)) return false;
  // smallest W with count_above(W) <= pos: the pos-th item is of class W - 1
  int lo = 1, hi = a.ctx_cap / U + 2;  // every item's class is at most ctx_cap / U + 1
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (count_above(mid) <= pos)
      hi = mid;
    else
      lo = mid + 1;
  }
  int r = pos - count_above(lo);  // rank among the items of class lo - 1
  const int nbits = 33 - __builtin_clz((unsigned)a.n_qtiles);
#pragma unroll
  for (int c = 0; c < kRankSeqChunks; ++c) {
    if (c < nchunks) {
      const int lo_c = above(lo, c);
      const int e = above(lo - 1, c) - lo_c;  // this lane's items of class lo - 1: qt in [nq - lo_c - e, nq - lo_c)
      const int pre = wave_prefix_bits(e, nbits);
      const int tot = wave_sum_bits(e, nbits);
      if (r < tot) {
        const unsigned long long hit = __builtin_amdgcn_ballot_w64(e > 0 && pre <= r && r < pre + e);
        const int l = (int)__builtin_ctzll(hit);
        const int qt = nq[c] - lo_c - 1 - (r - pre);  // the longest first
        seq_out = c * 64 + l;
        qt_out = __builtin_amdgcn_readlane(qt, l);
        return true;
      }
      r -= tot;
    }
  }
  return false;
}

template <int D, int DV, int G, bool kBs8>
__global__ void __launch_bounds__(kPrefillThreads, 2) prefill_chunk_kernel(const PrefillKernelArgs a) {
  using Sh = PrefillShape<G>;
  constexpr int GWH = Sh::GWH;
  constexpr int HALVES = Sh::HALVES;
  constexpr int QT = Sh::QT;
  using GK = TileGather<D, kPrefillWaves>;
  using GV = TileGather<DV, kPrefillWaves>;
  constexpr int NDS = D / 16;        // k-steps of Q K^T
  constexpr int NDT = DV / 32;       // 32-row tiles of O^T

  // kKBufs K tiles and kVBufs V tiles (80 KB at head dims 128: two
  // work-groups fill a CU's LDS).  At step t the waves read K of tile t+1
  // (scores) and V of tile t (P.V) while K of tile t+2 and V of tile t+1
  // are loaded; K of tile t stays for a redo.
  constexpr int kKTile = KT * D * 2, kVTile = KT * DV * 2;  // bytes
  constexpr int kVBase = kKBufs * kKTile;
  constexpr int kLdsBytes = kVBase + kVBufs * kVTile;
  __shared__ __attribute__((aligned(1024))) char lds[kLdsBytes];

  // Work id.  Work-groups are dispatched round-robin over the 8 XCDs; the
  // remap gives each XCD a contiguous range of work ids, ordered (kv head,
  // head part, dispatch position): each XCD serves whole kv heads, whose
  // items read the same K/V in its L2.
  const int nwg = (a.n_work + 7) & ~7;  // the grid: a multiple of 8
  const int bid = (int)__builtin_amdgcn_workgroup_id_x();
  const int wid = (bid & 7) * (nwg >> 3) + (bid >> 3);
  if (wid >= a.n_work) return;
  const int n_items = a.num_seqs * a.n_qtiles;
  const int pos = wid % n_items;
  const int half = (wid / n_items) % HALVES;
  const int kvh = wid / n_items / HALVES;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  int seq, qtile;
  if (a.num_seqs <= 64 * kRankSeqChunks) {
    if (!pick_item<QT>(a, pos, lane, seq, qtile)) return;
  } else {
    // plain order: each sequence's query tiles from the last
    seq = pos / a.n_qtiles;
    qtile = a.n_qtiles - 1 - pos % a.n_qtiles;
  }

  seq = __builtin_amdgcn_readfirstlane(seq);
  qtile = __builtin_amdgcn_readfirstlane(qtile);
  int r1 = min(a.query_start_loc[seq + 1], a.num_query_tokens);
  int r0 = a.query_start_loc[seq];
  r0 = max(0, min(r0, r1));
  const int q_len = r1 - r0;
  // the chunk ends the context
  int ctx = min(a.context_lens[seq], a.ctx_cap);
  ctx = max(ctx, 0);
  const int t_begin = qtile * QT;
  if (t_begin >= q_len) return;
  const int prefix = ctx - q_len;

  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hs = wave % GWH;           // head slot of this wave
  const int tg = wave / GWH;
  const int head = kvh * G + half * GWH + hs;  // the wave's query head
  const int tw0 = t_begin + tg * 32;   // first query of this wave
  const int col = lane & 31;
  const int hh = lane >> 5;
  const int t = tw0 + col;             // this lane's query (chunk row)
  const bool qvalid = t < q_len;
  // last key this lane's query sees: its position in the context
  const int qpos = prefix + t;
  // smallest of them in the wave: tiles past it need the mask
  int qpos_lo = qpos;
#pragma unroll
  for (int sft = 1; sft < 64; sft <<= 1) qpos_lo = min(qpos_lo, __shfl_xor(qpos_lo, sft));
  qpos_lo = __builtin_amdgcn_readfirstlane(qpos_lo);

  // Q of this lane's query (negated, exactly, under a negative scale; the
  // scores are then multiplied by |scale| * log2(e))
  const float sl = fabsf(a.scale_log2);
  const uint32_t qsign = a.scale_log2 < 0.f ? 0x80008000u : 0u;
  bf16x8_t qb[NDS];
  {
    const uint4 *qrow = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) +
                                                        ((size_t)(r0 + (qvalid ? t : 0)) * a.num_heads + head) * D);
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const uint4 w = qvalid ? qrow[ds * 2 + hh] : make_uint4(0, 0, 0, 0);
      qb[ds] = as_bf16x8(make_uint4(w.x ^ qsign, w.y ^ qsign, w.z ^ qsign, w.w ^ qsign));
    }
  }

  // keys this work-group needs: 0 .. (largest query position of the tile)
  const int t_last = min(t_begin + QT, q_len) - 1;
  int kend = max(0, min(ctx, prefix + t_last + 1));
  kend = __builtin_amdgcn_readfirstlane(kend);
  const int ntiles = (kend + KT - 1) / KT;

  const int shift = a.block_shift;
  const int bs_mask = (1 << shift) - 1;
  const uint32_t slot_stride = (uint32_t)a.num_kv_heads * D;  // elements between K slots
  const uint32_t vslot_stride = (uint32_t)a.num_kv_heads * DV;
  const uint32_t block_bytes = (slot_stride << shift) * 2u;
  const uint32_t vblock_bytes = (vslot_stride << shift) * 2u;
  const char *kbase = reinterpret_cast<const char *>(static_cast<const uint16_t *>(a.k_cache) + (size_t)kvh * D);
  const char *vbase = reinterpret_cast<const char *>(static_cast<const uint16_t *>(a.v_cache) + (size_t)kvh * DV);
  const char *zero = reinterpret_cast<const char *>(&kZeroChunk[0]);
  const int32_t *bt = a.block_tables + (size_t)seq * a.max_blocks_per_seq;
  const int max_blocks = a.max_blocks_per_seq;
  const int num_blocks = a.num_blocks;
  GK gk;
  GV gv;
  gk.init(wave, lane, bs_mask, slot_stride);
  gv.init(wave, lane, bs_mask, vslot_stride);
  // per-lane parts of the fragment addresses (see TileGather)
  const int k_even = ((hh ^ ((col >> 2) & 3)) << 4);
  const int k_odd = (((2 + hh) ^ ((col >> 2) & 3)) << 4);
  const int vg = lane >> 4, vs = lane & 15;
  const int v_lane = (4 * (vg >> 1) + (vs >> 2)) * 64 + (vs & 1) * 8;
  const int v_slot = 2 * (vg & 1) + ((vs >> 1) & 1);
  const int v_off0 = v_lane + ((v_slot ^ ((vg >> 1) & 3)) << 4);        // keys of the first read
  const int v_off1 = v_lane + 8 * 64 + ((v_slot ^ (((vg >> 1) + 2) & 3)) << 4);  // 8 keys further

  // running state of this lane's query: reference max m (base-2 units of
  // the scaled scores), nm = -m (0 while no key has been seen, m = -inf),
  // and the running sum l
  float m = -INFINITY, nm = 0.f, l = 0.f;
  f32x16_t o[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;

  typedef __attribute__((address_space(3))) const char *lds_cptr;
  const uint32_t sk_lds = (uint32_t)(size_t)((lds_cptr)(const char *)&lds[0]);
  const uint32_t sv_lds = sk_lds + (uint32_t)kVBase;
  auto ktile = [&](int j) { return reinterpret_cast<const uint16_t *>(&lds[(j % kKBufs) * kKTile]); };
  auto vtile = [&](int j) { return reinterpret_cast<const uint16_t *>(&lds[kVBase + (j % kVBufs) * kVTile]); };

  // raw scores S^T for keys k0 .. k0+63 (s[0]: first 32 keys, s[1]: last 32)
  auto qk = [&](const uint16_t *skb, f32x16_t (&s)[2]) {
    // chunk 2 ds + hh of keys col and 32 + col: group ds / 2, slot
    // (2 (ds % 2) + hh) ^ ((col / 4) % 4)
    typedef __attribute__((address_space(3))) const bf16x8_t *lds_frag_ptr;
    uint32_t ke = (uint32_t)(size_t)((lds_cptr)(const char *)skb + col * 64 + k_even);
    uint32_t ko = (uint32_t)(size_t)((lds_cptr)(const char *)skb + col * 64 + k_odd);
    asm volatile("" : "+v"(ke), "+v"(ko));
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const uint32_t p = ((ds & 1) ? ko : ke) + (ds / 2) * 4096;
      const bf16x8_t a0 = *(lds_frag_ptr)(size_t)(p);
      const bf16x8_t a1 = *(lds_frag_ptr)(size_t)(p + 2048);
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qb[ds], ds == 0 ? f32x16_t{} : s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qb[ds], ds == 0 ? f32x16_t{} : s[1], 0, 0, 0);
    }
  };

  // O^T += V^T P^T; the A operand takes the same keys from row d of V^T.
  // It comes from transposing LDS reads of the row-major V tile: in each
  // 16-lane group, source lane s reads 4 d-values of one key (key K0 + s/4,
  // d = D0 + 4 (s%4)) and lane o receives d = D0 + o of keys K0 .. K0+3;
  // two reads give the 8 keys of the B operand's k-step.  Lane s of 16-lane
  // group g reads, for tile dt and k-step ks, key (ks / 2) 32 + (ks % 2) 16
  // + 4 (g / 2) + s / 4 (+8 for the second read), slot (2 (g % 2) + (s / 2)
  // % 2) ^ ((key / 4) % 4), half s % 2 (address arithmetic in the LDS
  // address space, constants last, so that they fold into the
  // instructions' offset fields)
  auto pv = [&](const uint16_t *svb, const bf16x8_t (&pb)[4]) {
    typedef short v4s __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4s *lds_v4s_ptr;
    // the two per-lane bases pass through an empty asm statement: opaque
    // vector values, so that base + constant selects the instructions'
    // offset field instead of a separate address per read
    uint32_t va0 = (uint32_t)(size_t)((lds_cptr)(const char *)svb + v_off0);
    uint32_t va1 = (uint32_t)(size_t)((lds_cptr)(const char *)svb + v_off1);
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
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pb[ks], o[dt], 0, 0, 0);
      }
    }
  };

  // weights of one tile, 2^(s * scale - m) from raw scores s (raw) or 2^s
  // from exponents already relative to the reference, bf16 in the B layout
  // of the P.V products, and their sum over this lane's keys; the running
  // sum takes the same bf16 weights that multiply V, two at a time
  // (v_dot2_f32_bf16 against ones), so numerator and denominator agree
  auto weights = [&](f32x16_t (&s)[2], bf16x8_t (&pb)[4], bool raw) -> float {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[0][r] = fast_exp2(raw ? fmaf(s[0][r], sl, nm) : s[0][r]);
      s[1][r] = fast_exp2(raw ? fmaf(s[1][r], sl, nm) : s[1][r]);
    }
    // P^T in the B layout: k-step (sub-tile st, half u) = registers
    // 8u..8u+7 of s[st], i.e. keys st*32 + 16u + 8*(e/4) + 4*hh + e%4
    pb[0] = pack8(s[0], 0);
    pb[1] = pack8(s[0], 8);
    pb[2] = pack8(s[1], 0);
    pb[3] = pack8(s[1], 8);
    float ps = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint4 w = __builtin_bit_cast(uint4, pb[u]);
      ps = dot2_bf16(w.x, kBf16PairOnes, ps);
      ps = dot2_bf16(w.y, kBf16PairOnes, ps);
      ps = dot2_bf16(w.z, kBf16PairOnes, ps);
      ps = dot2_bf16(w.w, kBf16PairOnes, ps);
    }
    return ps;
  };

  // New reference from the exponents of one tile (s = scaled scores + nm):
  // the lane's max over both halves of the wave; when it exceeds m by more
  // than the slack (always on the first tile with a key), O and l are
  // rescaled and nm changes by d, which is returned (0 when it stays).
  auto new_reference = [&](const f32x16_t (&s)[2]) -> float {
    float rmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) rmax = fmaxf(fmaxf(rmax, s[0][r]), s[1][r]);
    const float tmax = xor32_max(rmax) - nm;  // -inf when no key of the tile is seen
    const bool grow = tmax > m + kRescaleSlack;
    float d = 0.f;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float m_new = grow ? tmax : m;
      const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - m_new);
      const float nm_new = (m_new == -INFINITY) ? 0.f : -m_new;
      d = nm_new - nm;
      m = m_new;
      nm = nm_new;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    }
    return d;
  };

  // leading tiles every query of this wave sees whole: no mask, no max
  const int n_plain = min(ntiles, max(0, (qpos_lo + 1) / KT));

  // loads of tile j, K into buffer j % kKBufs and V into buffer j % kVBufs
  auto gather_k = [&](int j, const TileIds &ids) {
    const int k0 = j * KT;
    const uint32_t dk = sk_lds + (uint32_t)((j % kKBufs) * kKTile);
    if (k0 + KT <= kend)
      gk.issue(kBs8, false, dk, ids, kbase, zero, num_blocks, block_bytes, k0, kend, lane);
    else
      gk.issue(kBs8, true, dk, ids, kbase, zero, num_blocks, block_bytes, k0, kend, lane);
  };
  auto gather_v = [&](int j, const TileIds &ids) {
    const int k0 = j * KT;
    const uint32_t dv = sv_lds + (uint32_t)((j % kVBufs) * kVTile);
    if (k0 + KT <= kend)
      gv.issue(kBs8, false, dv, ids, vbase, zero, num_blocks, vblock_bytes, k0, kend, lane);
    else
      gv.issue(kBs8, true, dv, ids, vbase, zero, num_blocks, vblock_bytes, k0, kend, lane);
  };
  // K and V rows of one key share the block, and a wave's K and V loads
  // cover the same 16 keys, so one read of block ids serves both
  auto tile_ids = [&](int j) { return gk.ids(kBs8, bt, j * KT, shift, max_blocks); };

  // Pipeline, one barrier per step t:
  //   loads of K(t+2) and V(t+1) issued;  S(t+1) = K(t+1) Q^T;  weights of
  //   S(t);  O += V(t) P(t);  block ids of tile t+3 read;  wait for this
  //   wave's loads;  barrier.
  // ids1 holds the block ids of tile t+1, ids2 those of tile t+2.
  TileIds ids1 = tile_ids(0);
  gather_k(0, ids1);
  gather_v(0, ids1);
  ids1 = tile_ids(1);
  gather_k(1, ids1);
  TileIds ids2 = tile_ids(2);
  wait_vmcnt<0>();
  __syncthreads();

  f32x16_t sa[2], sb[2];  // scores of two consecutive tiles (ping-pong)
  qk(ktile(0), sa);

  // one step on tile j whose scores are in cur; the next tile's go to nxt.  kFull: causal mask where the tile crosses the diagonal, and
  // the tile's max (first tile, diagonal tiles); otherwise no mask and no
  // max, with the sum check.
  auto step = [&](bool kFull, int j, f32x16_t (&cur)[2], f32x16_t (&nxt)[2]) __attribute__((always_inline)) {
    const int k0 = j * KT;
    gather_k(j + 2, ids2);
    gather_v(j + 1, ids1);
    if (kFull) {
      // exponents relative to the reference; causal mask on tiles that
      // cross this wave's diagonal (register r of this lane holds key
      // 8*(r/4) + 4*hh + r%4)
      const bool diag = k0 + KT - 1 > qpos_lo;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = 8 * (r >> 2) + 4 * hh + (r & 3);
        cur[0][r] = (!diag || k0 + kr <= qpos) ? fmaf(cur[0][r], sl, nm) : -INFINITY;
        cur[1][r] = (!diag || k0 + 32 + kr <= qpos) ? fmaf(cur[1][r], sl, nm) : -INFINITY;
      }
      const float d = new_reference(cur);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        cur[0][r] += d;
        cur[1][r] += d;
      }
    }
    // From here to the P.V products the code is one basic block: the
    // scores of the next tile (independent of this tile's weights; past the
    // last tile the buffer holds zero rows and the result is not used) are
    // interleaved with the exponentials, so the matrix and vector units
    // work at the same time.
    qk(ktile(j + 1), nxt);
    bf16x8_t pb[4];
    float ps = weights(cur, pb, !kFull);
    if (!kFull) {
      if (__builtin_amdgcn_ballot_w64(ps > kSumLimit)) {
        // a score far above the reference: redo this tile's scores and
        // move the reference (the tile is still in LDS)
        qk(ktile(j), cur);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          cur[0][r] = fmaf(cur[0][r], sl, nm);
          cur[1][r] = fmaf(cur[1][r], sl, nm);
        }
        const float d = new_reference(cur);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          cur[0][r] += d;
          cur[1][r] += d;
        }
        ps = weights(cur, pb, false);
      }
    }
    l += ps;
    pv(vtile(j), pb);
    ids1 = ids2;
    ids2 = tile_ids(j + 3);
    wait_vmcnt<0>();  // this wave's loads of K(j+2) and V(j+1) are in LDS
    __syncthreads();
  };

  constexpr bool full = true, plain = false;
  int j = 0;
  if (ntiles > 0) {
    step(full, 0, sa, sb);
    j = 1;
    // plain tiles, two per iteration so that the score registers alternate
    for (; j + 1 < n_plain; j += 2) {
      step(plain, j, sb, sa);
      step(plain, j + 1, sa, sb);
    }
    if (j < n_plain) {
      step(plain, j, sb, sa);
      ++j;
#pragma unroll
      for (int s = 0; s < 2; ++s) sb[s] = sa[s];
    }
    for (; j < ntiles; ++j) {
      step(full, j, sb, sa);
#pragma unroll
      for (int s = 0; s < 2; ++s) sb[s] = sa[s];
    }
  }

  const float lsum = xor32_sum(l);  // cross-lane: before the divergent store
  if (qvalid) {
    uint16_t *orow = static_cast<uint16_t *>(a.out) + ((size_t)(r0 + t) * a.num_heads + head) * DV;
    // one division per row, then a multiply per element (an IEEE division
    // per element is ~10 vector instructions)
    const float inv = (lsum > 0.f) ? 1.f / lsum : 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const int d0 = dt * 32 + 8 * rq + 4 * hh;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = o[dt][4 * rq + e] * inv;
        *reinterpret_cast<uint2 *>(orow + d0) = make_uint2(pack_bf16x2_rne(v[0], v[1]), pack_bf16x2_rne(v[2], v[3]));
      }
  }
}

template <int D, int DV, int G>
static hipError_t launch_t(const PrefillArgs &a, hipStream_t stream) {
  const bool bs8 = a.cache.block_size == 8;
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
  const int64_t n_work = (int64_t)a.num_seqs * a.cache.num_kv_heads * Sh::HALVES * k.n_qtiles;
  if (n_work <= 0) return hipSuccess;
  if (n_work > (int64_t)0x7fffffff - 8) return hipErrorInvalidConfiguration;
  k.n_work = (int)n_work;
  k.scale_log2 = a.scale * kLog2e;
  const unsigned grid = (unsigned)((n_work + 7) / 8 * 8);
  if (bs8)
    hipLaunchKernelGGL((prefill_chunk_kernel<D, DV, G, true>), dim3(grid), dim3(kPrefillThreads), 0, stream, k);
  else
    hipLaunchKernelGGL((prefill_chunk_kernel<D, DV, G, false>), dim3(grid), dim3(kPrefillThreads), 0, stream, k);
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
