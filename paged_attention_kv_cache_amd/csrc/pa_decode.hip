// Paged decode attention: one query token per sequence against its whole
// context in the block-table KV cache, with optional split-K
// (flash-decoding) partitions and a reduce kernel.
//
// What is computed: TensorSharp, Mistral 3 page, section 3 "Forward graph".
// The newest token's K/V are already in the cache; scores
// s_p = scale * q.k_p for every context position p; softmax over p; the
// weighted sum of V.  Query head h reads kv head h / G (GQA, section 4.1).
// The paged layout and the online-softmax loop parallel over (sequence,
// head) are from section 11 "Batched / paged forward".
//
// How it maps to gfx950.  Two partition kernels share the grid shape,
// the split-K partials and the reduce kernel:
//  * bf16 pools (the serving path): decode_partition_mfma_kernel
//    (Bf16DecodeMfma, below).  One wave per kv head, a work-group per (4
//    kv heads, sequence, partition).  Per tile of 16 tokens the scores of
//    the kv head's G query heads and their weighted V rows are two small
//    MFMA products, so the vector work per token does not grow with G.
//    K/V rows are loaded into registers and staged through the wave's own
//    LDS slice; the next tile's loads are in flight while a staged tile is
//    computed.
//  * fp32 pools: decode_partition_kernel (the generic kernel next).  One
//    work-group (4 waves) per (partition, kv head, sequence) owns the G
//    query heads of that kv head, so each K/V byte of the partition is read
//    once for all G heads.  A token's K row is read by L = row_bytes / 16
//    lanes with one 128-bit load each (64 / L tokens per load instruction,
//    kUnroll loads of K and of V in flight per lane); the q.k partial sums
//    are reduced across the L lanes with DPP, and the L lanes of a token's
//    K row also cover its V row (DV / L elements each), so key and value
//    head dims may differ (section 4.1 of the same page).  Each wave runs
//    its own online softmax over its chunks and the four waves merge
//    (m, l, o) through LDS.
//  * In both, scores are kept in base-2 units (scale * log2(e)), so one
//    v_exp_f32 gives each weight, and a token outside the context or in an
//    invalid block is *selected out*: its score is -inf, its weight exactly
//    0, and its V row never enters a product, so stale or NaN pool contents
//    cannot leak in.  Every load covers consecutive tokens inside one
//    block, so block-table reads are scalar loads.  A sequence that fits in
//    one partition is normalised and stored directly; otherwise the
//    partition's (m, l, o) go to the workspace and the reduce kernel merges
//    the partitions.
#include <type_traits>

#include "pa_common.h"

namespace pa {

template <typename T, int D>
struct DecodeShape {
  static constexpr int kElems = Chunk<T>::kElems;         // elements per 16-byte chunk
  static constexpr int kLanesPerRow = D / kElems;         // lanes sharing one token row
  static constexpr int kRowsPerWave = 64 / kLanesPerRow;  // tokens per load instruction
  static constexpr int kUnroll = 8;                       // K (and V) loads in flight per lane
  static constexpr int kChunk = kRowsPerWave * kUnroll;   // tokens per wave step
  static constexpr int kWaves = 4;
  static constexpr int kThreads = 64 * kWaves;
  static_assert(kThreads == 256, "launch bounds assume 256 threads");
  static_assert(kLanesPerRow >= 8 && kLanesPerRow <= 32, "unsupported row width");
};

struct DecodeKernelArgs {
  void *out;
  const void *q;
  const void *k_cache;
  const void *v_cache;
  const int32_t *block_tables;
  const int32_t *context_lens;
  float *ws_m;
  float *ws_l;
  float *ws_o;
  int num_heads;
  int num_kv_heads;
  int num_blocks;
  int block_shift;       // log2(block_size)
  int max_blocks_per_seq;
  int ctx_cap;           // min(max_context_len, max_blocks_per_seq * block_size)
  int partition_size;    // tokens per partition; 0 = whole context
  int max_partitions;
  int num_seqs;
  float scale_log2;      // scale * log2(e)
  // cascade: rows group_start[g] .. group_start[g+1]-1 share their first
  // shared_len[g] tokens (partial in slot 0); NULL for plain decode
  const int32_t *group_start;
  const int32_t *shared_len;
  int num_groups;
  int shared_chunk;      // the shared part's partials: slots 0 .. ceil(shared / shared_chunk) - 1
  int shared_chunks;     // cascade: chunks per group this launch computes
  int shared_cap;        // shared tokens are clamped to this (the chunks launched)
  int shared_items;      // cascade: launch items of the shared chunks (0: none in this launch)
  int shared_stride;     // cascade: items between the column tiles of one shared chunk
  int col_tiles;         // cascade: 16-column tiles per group, ceil(max_group_size * G / 16)
  // prefill rows (non-NULL): index r of the generic kernel is packed query
  // row r of sequences 0 .. num_prefill_seqs-1 (see decode_row)
  const int32_t *query_start_loc;
  int num_prefill_seqs;
  // fused append (non-NULL): newest tokens' K and V rows, [S, Hkv, D]
  const void *new_k;
  const void *new_v;
};

__device__ __forceinline__ int decode_context(const DecodeKernelArgs &a, int seq) {
  int ctx = a.context_lens[seq];
  ctx = ctx < a.ctx_cap ? ctx : a.ctx_cap;
  return ctx > 0 ? ctx : 0;
}

__device__ __forceinline__ int decode_num_partitions(const DecodeKernelArgs &a, int ctx) {
  if (a.partition_size <= 0 || ctx <= 0) return 1;
  return (ctx + a.partition_size - 1) / a.partition_size;
}

// Row r of the generic kernel: the block-table row it reads and the keys
// it sees.  Decode: sequence r, its whole context.  Prefill rows: the
// sequence i that owns packed query row r, and the keys up to that row's
// own position context_lens[i] - q_len_i + (r - query_start_loc[i]) (the
// chunk ends its context).  Returns false for a row that no sequence owns
// (it is left untouched).
__device__ __forceinline__ bool decode_row(const DecodeKernelArgs &a, int r, int &tab_row, int &ctx) {
  if (!a.query_start_loc) {
    tab_row = r;
    ctx = decode_context(a, r);
    return true;
  }
  const int32_t *qsl = a.query_start_loc;
  tab_row = 0;
  ctx = 0;
  if (a.num_prefill_seqs <= 0 || r < max(qsl[0], 0) || r >= qsl[a.num_prefill_seqs]) return false;
  int lo = 0, hi = a.num_prefill_seqs - 1;  // the i with qsl[i] <= r < qsl[i+1]
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (qsl[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  const int q_len = qsl[lo + 1] - qsl[lo];
  const int full = decode_context(a, lo);
  const int n = full - q_len + (r - qsl[lo]) + 1;  // at most `full` for an ascending query_start_loc
  tab_row = lo;
  ctx = max(0, min(n, full));
  return true;
}

// cascade: the shared tokens of a row's group (0 outside cascade), at most
// its context
__device__ __forceinline__ int decode_shared(const DecodeKernelArgs &a, int seq, int ctx) {
  if (!a.group_start) return 0;
  int lo = 0, hi = a.num_groups - 1;  // the group g with group_start[g] <= seq
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.group_start[mid] <= seq) lo = mid;
    else hi = mid - 1;
  }
  return max(0, min(min(a.shared_len[lo], a.shared_cap), ctx));
}

template <typename T>
__device__ __forceinline__ void store_one(void *base, size_t idx, float v);
template <>
__device__ __forceinline__ void store_one<float>(void *base, size_t idx, float v) {
  static_cast<float *>(base)[idx] = v;
}
template <>
__device__ __forceinline__ void store_one<bf16_t>(void *base, size_t idx, float v) {
  static_cast<uint16_t *>(base)[idx] = (uint16_t)f32_to_bf16_bits(v);
}

template <typename T, int D, int DV, int G>
__global__ void __launch_bounds__(256)
decode_partition_kernel(const DecodeKernelArgs a) {
  using S = DecodeShape<T, D>;
  constexpr int E = S::kElems;
  constexpr int EV = DV / S::kLanesPerRow;  // V elements per lane
  using VRow = Vec<T, EV>;
  constexpr int L = S::kLanesPerRow;
  constexpr int R = S::kRowsPerWave;
  constexpr int U = S::kUnroll;
  constexpr int CH = S::kChunk;
  constexpr int W = S::kWaves;

  const int part = blockIdx.x;
  const int kvh = blockIdx.y;
  const int seq = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row = lane / L;
  const int col = lane % L;

  int tab_row, ctx;
  if (!decode_row(a, seq, tab_row, ctx)) return;
  const int nparts = decode_num_partitions(a, ctx);
  if (part >= nparts) return;
  const int ps = a.partition_size > 0 ? a.partition_size : ctx;
  const int p0 = part * ps;
  const int p1 = min(ctx, p0 + ps);

  // q of the G heads of this kv head, this lane's 16-byte slice of D,
  // pre-multiplied by scale * log2(e).
  float qf[G][E];
  {
    const uint4 *qv = reinterpret_cast<const uint4 *>(
        static_cast<const T *>(a.q) + ((size_t)seq * a.num_heads + (size_t)kvh * G) * D);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const uint4 c = qv[h * L + col];
      Chunk<T>::widen(c, qf[h]);
#pragma unroll
      for (int e = 0; e < E; ++e) qf[h][e] *= a.scale_log2;
    }
  }

  const size_t slot_stride = (size_t)a.num_kv_heads * D;  // elements between K slots
  const size_t vslot_stride = (size_t)a.num_kv_heads * DV;
  const T *kbase = static_cast<const T *>(a.k_cache) + (size_t)kvh * D + col * E;
  const T *vbase = static_cast<const T *>(a.v_cache) + (size_t)kvh * DV + col * EV;
  const int32_t *bt = a.block_tables + (size_t)tab_row * a.max_blocks_per_seq;
  const int bs_mask = (1 << a.block_shift) - 1;

  float m_run[G], l_run[G], acc[G][EV];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EV; ++e) acc[h][e] = 0.f;
  }

  const int ntok = p1 - p0;
  const int nchunks = ntok > 0 ? (ntok + CH - 1) / CH : 0;
  for (int c = wave; c < nchunks; c += W) {
    const int cbase = p0 + c * CH;
    uint4 kr[U];
    VRow vr[U];
    bool valid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tok0 = cbase + u * R;  // first token of this load, same for the wave
      const int tok = tok0 + row;
      int blk = -1;
      if (tok0 < p1) blk = bt[tok0 >> a.block_shift];
      valid[u] = (tok < p1) && ((unsigned)blk < (unsigned)a.num_blocks);
      kr[u] = make_uint4(0, 0, 0, 0);
      vr[u].zero();
      if (valid[u]) {
        const size_t slot = ((size_t)blk << a.block_shift) + (tok & bs_mask);
        kr[u] = *reinterpret_cast<const uint4 *>(kbase + slot * slot_stride);
        vr[u].load(vbase + slot * vslot_stride);
      }
    }

    // scores (base-2 units) for this lane's row token of every load
    float s[U][G];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[E];
      Chunk<T>::widen(kr[u], kf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) dot = fmaf(qf[h][e], kf[e], dot);
        dot = group_sum<L>(dot);
        s[u][h] = valid[u] ? dot : -INFINITY;
      }
    }

    // online softmax update over the chunk
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float cm = s[0][h];
#pragma unroll
      for (int u = 1; u < U; ++u) cm = fmaxf(cm, s[u][h]);
      cm = across_groups_max<L>(cm);
      const float m_new = fmaxf(m_run[h], cm);
      const float alpha = (m_new == -INFINITY) ? 1.f : fast_exp2(m_run[h] - m_new);
      m_run[h] = m_new;
      l_run[h] *= alpha;
#pragma unroll
      for (int e = 0; e < EV; ++e) acc[h][e] *= alpha;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[EV];
      vr[u].widen(vf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = valid[u] ? fast_exp2(s[u][h] - m_run[h]) : 0.f;
        l_run[h] += p;
#pragma unroll
        for (int e = 0; e < EV; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
      }
    }
  }

  // sum the rows of the wave (m is already uniform over the wave)
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l_run[h] = across_groups_sum<L>(l_run[h]);
#pragma unroll
    for (int e = 0; e < EV; ++e) acc[h][e] = across_groups_sum<L>(acc[h][e]);
  }

  __shared__ float sm_m[W][G];
  __shared__ float sm_l[W][G];
  __shared__ float sm_o[W][G][DV];
  if (lane < L) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EV; ++e) sm_o[wave][h][col * EV + e] = acc[h][e];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sm_m[wave][h] = m_run[h];
      sm_l[wave][h] = l_run[h];
    }
  }
  __syncthreads();

  const bool direct = (nparts == 1);
  for (int i = threadIdx.x; i < G * DV; i += S::kThreads) {
    const int h = i / DV;
    const int d = i - h * DV;
    float M = sm_m[0][h];
#pragma unroll
    for (int w = 1; w < W; ++w) M = fmaxf(M, sm_m[w][h]);
    float o = 0.f, l = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float mw = sm_m[w][h];
        const float f = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
        o = fmaf(sm_o[w][h][d], f, o);
        l = fmaf(sm_l[w][h], f, l);
      }
    }
    const int head = kvh * G + h;
    if (direct) {
      const float r = (l > 0.f) ? o / l : 0.f;
      store_one<T>(a.out, ((size_t)seq * a.num_heads + head) * DV + d, r);
    } else {
      const size_t idx = ((size_t)seq * a.num_heads + head) * a.max_partitions + part;
      a.ws_o[idx * DV + d] = o;
      if (d == 0) {
        a.ws_m[idx] = M;
        a.ws_l[idx] = l;
      }
    }
  }
}

// ------------------------------------------------------------------------
// Shared by the bf16 partition kernel below.
constexpr int kDecodeWaves = 4;  // waves per work-group
// Grid order of the bf16 partition kernel: kv head group fastest, then the
// (sequence, partition) pairs by size: every full partition first, then
// the partial last partitions, longest first, so that the work-groups
// dispatched last are the short ones (batches of at most 64 sequences;
// larger ones, and cascade launches, take sequence then partition, so that
// the partitions that exist for every sequence are dispatched first and
// the empty ones past short contexts come last).

// A wave rescales its running sums only when a head's max grows by more
// than this many base-2 units; until then the weights exp2(s - m) may reach
// 2^8, which the fp32 sums and the bf16 weights hold exactly as well.
constexpr float kDecodeRescaleSlack = 8.f;

// Read-only view for inputs that no work-group writes during a launch
// (block tables, context lengths): loads through the constant address
// space stay scalar for wave-uniform indices even after the kernel's own
// stores and fences.
typedef const __attribute__((address_space(4))) int32_t *ro_i32_ptr;
__device__ __forceinline__ ro_i32_ptr read_only(const int32_t *p) { return (ro_i32_ptr)(p); }

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// Dispatch order by size.  The (sequence, partition) pairs of a batch of at
// most 64 sequences are numbered so that every full partition comes first
// (partition-major), then the partial last partitions, longest first (ties
// by sequence; the single empty partition of a sequence with no context
// counts as a partial one of length 0); work-group item i takes pair i.  Computed by one wave, lane
// s holding sequence s.  Returns false for an item past the last pair.
__device__ __forceinline__ bool size_order_item(const DecodeKernelArgs &a, int item, int lane, int &seq_out,
                                                int &part_out) {
  const int S = a.num_seqs;
  const int ps = a.partition_size;
  // the tokens a row's partitions cover: its context, or (cascade) the
  // part of it after its shared tokens
  int ctx = lane < S ? decode_context(a, lane) : 0;
  if (a.group_start && lane < S) ctx -= decode_shared(a, lane, ctx);
  const int nfull = ctx / ps;
  const int rem = ctx - nfull * ps;
  // full pairs: cum(p) = sum_s min(nfull_s, p) pairs come before partition p
  auto cum = [&](int p) {
    int v = min(nfull, p);
#pragma unroll
    for (int sft = 1; sft < 64; sft <<= 1) v += __shfl_xor(v, sft);
    return v;
  };
  // lane p holds cum(p) (up to 64 partitions): one pass over the
  // sequences' counts in scalar registers instead of a cross-lane sum per
  // step of a search
  int cum_l = 0, total_full = 0;
  if (a.max_partitions <= 64) {
    for (int s = 0; s < S; ++s) {
      const int nf = __builtin_amdgcn_readlane(nfull, s);
      cum_l += min(nf, lane);
      total_full += nf;
    }
  } else {
    total_full = cum(a.max_partitions);
  }
  if (item < total_full) {
    int lo;  // the p with cum(p) <= item < cum(p+1)
    int k;
    if (a.max_partitions <= 64) {
      lo = __builtin_popcountll(__builtin_amdgcn_ballot_w64(lane < a.max_partitions && cum_l <= item)) - 1;
      k = item - __builtin_amdgcn_readlane(cum_l, lo);
    } else {
      lo = 0;
      int hi = a.max_partitions - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cum(mid) <= item) lo = mid;
        else hi = mid - 1;
      }
      k = item - cum(lo);
    }
    const unsigned long long has = __builtin_amdgcn_ballot_w64(nfull > lo);
    const int rank = __builtin_amdgcn_mbcnt_hi((unsigned)(has >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)has, 0));
    const unsigned long long hit = __builtin_amdgcn_ballot_w64(nfull > lo && rank == k);
    if (hit == 0) return false;
    seq_out = __builtin_ctzll(hit);
    part_out = lo;
    return true;
  }
  // partial pairs: a last partition shorter than ps, or the one empty
  // partition of a sequence with no context (its output row is zero)
  const bool partial = lane < S && (rem > 0 || ctx == 0);
  const unsigned long long has = __builtin_amdgcn_ballot_w64(partial);
  const int j = item - total_full;
  int rank = 0;  // among partial pairs: longer first, then lower sequence
  for (int s = 0; s < S; ++s) {
    const int r = __builtin_amdgcn_readlane(rem, s);
    rank += ((has >> s) & 1) && (r > rem || (r == rem && s < lane)) ? 1 : 0;
  }
  const unsigned long long hit = __builtin_amdgcn_ballot_w64(partial && rank == j);
  if (hit == 0) return false;
  seq_out = __builtin_ctzll(hit);
  part_out = __builtin_amdgcn_readlane(nfull, seq_out);
  return true;
}

// ------------------------------------------------------------------------
// Matrix-core decode (bf16).  Per kv head, the scores of a tile of 16
// tokens and the tile's share of the weighted sum are two small matrix
// products:
//   S^T = K Q^T    on v_mfma_f32_16x16x32_bf16 (16 tokens x 16 columns, the
//                  G query heads of the kv head as columns, the rest zero),
//   O^T += V^T P^T on v_mfma_f32_16x16x16_bf16 (value dims x columns).
// In the accumulator layout lane l holds column l % 16 and tokens
// 4 (l / 16) .. 4 (l / 16) + 3 of S^T, which is also the B operand layout
// of the second product, so the weights go from the exponentials straight
// into the products.  The vector work per token (a scale, an exponential,
// the max and the sum, shared by up to 16 heads) does not grow with G.
//  * One wave per kv head: a work-group (4 waves) covers 4 consecutive kv
//    heads of one (sequence, partition), every wave all of the partition's
//    tokens; no cross-wave merge.
//  * A tile is loaded row-major, 64 / (D/8) tokens x the kv head's K row
//    per load instruction (and likewise for V rows of DV elements): a
//    scalar block id per instruction, since tiles start at a multiple of 8
//    tokens and blocks hold 8, 16 or 32.  The rows go into registers, from
//    there into the wave's own LDS slice; the registers then take the next
//    tile's loads, which are in flight while the staged tile is computed.
//    One register set per wave leaves room for four work-groups per CU.
//    The score product reads K from LDS with one 16-byte read per lane and
//    k-step, the value product V^T with gfx950's transposing 8-byte reads.
//    Rows are padded (2D + 16 and 2DV + 32 bytes) so that both kinds of
//    reads hit distinct banks.
//  * Tokens outside the range, or in a block outside the pool, are
//    selected out: score -inf, weight 0, and their V rows zeroed before
//    they enter the product, whatever the slot holds.  (The cascade's
//    own-token ranges start anywhere: their first tile starts at the
//    multiple of 8 below and masks the tokens before the range.)
//  * The running max is a reference moved only when a tile exceeds it by
//    more than 2^8 (the rescale of l and O is then rare; exact in real
//    arithmetic, like an eager rescale); the running sum takes the fp32
//    weights, the products their bf16 roundings (nearest even).
//  * Fused append: the newest token's rows come from the input rows (they
//    replace the loaded slot contents in registers) and are written into
//    its slot after the last tile.
//  * Cascade decode's shared chunks run on the same products with other
//    columns: column j is query head j % G of member j / G of a group's
//    16/G-member column tile, each column with a key limit of its own
//    (decode_shared_chunk).
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4_t *lds_u4_ptr;
typedef __attribute__((address_space(3))) const bf16x8_t *lds_b8_ptr;
typedef __attribute__((address_space(3))) v4i16_t *lds_v4_ptr;

template <int D, int DV, int G>
struct Bf16DecodeMfma {
  static constexpr int TT = 16;             // tokens per tile
  static constexpr int LK = D / 8;          // lanes per K row (16 bytes each)
  static constexpr int LV = DV / 8;         // lanes per V row
  static constexpr int RK = 64 / LK;        // tokens per K load instruction (4 or 8)
  static constexpr int RV = 64 / LV;        // tokens per V load instruction
  static constexpr int NLK = TT / RK;       // K loads per tile
  static constexpr int NLV = TT / RV;       // V loads per tile
  static constexpr int NKS = D / 32;        // k-steps of the score product
  static constexpr int NDT = DV / 16;       // 16-row tiles of O^T
  static constexpr int KROW = 2 * D + 16;   // LDS bytes per K row: 16 rows at one chunk cover every bank
  static constexpr int VROW = 2 * DV + 32;  // LDS bytes per V row: the transposing reads of 8 rows cover every bank
  static constexpr int KBYTES = TT * KROW;
  static constexpr int LDS_BYTES = KBYTES + TT * VROW;  // one wave's slice
  static_assert((D == 64 || D == 128) && (DV == 64 || DV == 128), "head dims 64 or 128");
  static_assert(G >= 1 && G <= 16, "the query heads of a kv head are columns of a 16-wide tile");

  // One tile's rows: K load j holds tokens t0 + RK j .. (lane l: token
  // t0 + RK j + l / LK, 16-byte chunk l % LK of its row), V load j tokens
  // t0 + RV j ..; bit q of ok: tokens t0 + 4q .. t0 + 4q + 3 lie in a block
  // inside the pool.
  struct Tile {
    uint4 k[NLK];
    uint4 v[NLV];
    int ok;
  };

  // Addressing shared by a wave's loads: the table row, the pool bases,
  // the bytes per token slot, and this lane's byte offset (its token in the
  // load times the slot size, plus its kv head's row and its chunk).
  struct Rows {
    ro_i32_ptr tab;
    const char *kbase, *vbase;
    size_t kslot, vslot;
    uint32_t klane, vlane;
  };

  __device__ static __forceinline__ void issue(const DecodeKernelArgs &a, const Rows &w, int t0, int p1, Tile &t) {
    const int shift = a.block_shift;
    const int bs_mask = (1 << shift) - 1;
    int blk[TT / 4];
#pragma unroll
    for (int q = 0; q < TT / 4; ++q) blk[q] = w.tab[min((t0 + 4 * q) >> shift, a.max_blocks_per_seq - 1)];
    int ok = 0;
    size_t slot[TT / 4];
#pragma unroll
    for (int q = 0; q < TT / 4; ++q) {
      const bool good = (unsigned)blk[q] < (unsigned)a.num_blocks;
      ok |= good ? (1 << q) : 0;
      // a token past the range or in a block outside the pool reads the
      // pool's first slots
      slot[q] = (good && t0 + 4 * q < p1) ? ((size_t)(uint32_t)blk[q] << shift) + (size_t)((t0 + 4 * q) & bs_mask) : 0;
    }
#pragma unroll
    for (int j = 0; j < NLK; ++j) {
      const u32x4_t x = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t *>(w.kbase + slot[j * RK / 4] * w.kslot + w.klane));
      t.k[j] = make_uint4(x.x, x.y, x.z, x.w);
    }
#pragma unroll
    for (int j = 0; j < NLV; ++j) {
      const u32x4_t x = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t *>(w.vbase + slot[j * RV / 4] * w.vslot + w.vlane));
      t.v[j] = make_uint4(x.x, x.y, x.z, x.w);
    }
    t.ok = ok;
  }

  // Per-wave state.
  struct State {
    bf16x8_t qf[NKS];  // Q^T fragments: column l % 16, chunk 4 ks + l / 16 of that head's row
    f32x4_t o[NDT];    // O^T: column l % 16, value dims 16 dt + 4 (l / 16) + r
    float m, l;        // reference max (base-2 units) and this lane's part of the running sum
  };

  // The loaded tile at tokens t0 .. into the wave's LDS slice (row-major,
  // padded rows).  Rows of tokens outside [p0, p1) or in a block outside
  // the pool get a zero V row; the appended token's rows come from the
  // input.
  __device__ static __forceinline__ void stage(Tile &t, int t0, int p0, int p1, int pnew, uint4 kn, uint4 vn,
                                               int lane, uint32_t lds) {
    const int tk = lane / LK, ck = lane % LK;  // this lane's token in a K load, and its chunk
    const int tv = lane / LV, cv = lane % LV;
    if (t.ok != (1 << (TT / 4)) - 1 || t0 < p0 || t0 + TT > p1) {
#pragma unroll
      for (int j = 0; j < NLV; ++j) {
        const int tl = RV * j + tv;
        if (!(((t.ok >> (tl >> 2)) & 1) && t0 + tl >= p0 && t0 + tl < p1)) t.v[j] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    if (pnew >= t0 && pnew < t0 + TT && ((t.ok >> ((pnew - t0) >> 2)) & 1)) {
      const int tl = pnew - t0;
#pragma unroll
      for (int j = 0; j < NLK; ++j)
        if (j == tl / RK && tk == tl % RK) t.k[j] = kn;
#pragma unroll
      for (int j = 0; j < NLV; ++j)
        if (j == tl / RV && tv == tl % RV) t.v[j] = vn;
    }
    const uint32_t kw = lds + (uint32_t)(tk * KROW + ck * 16);
    const uint32_t vw = lds + (uint32_t)(KBYTES + tv * VROW + cv * 16);
#pragma unroll
    for (int j = 0; j < NLK; ++j)
      *(lds_u4_ptr)(size_t)(kw + j * RK * KROW) = u32x4_t{t.k[j].x, t.k[j].y, t.k[j].z, t.k[j].w};
#pragma unroll
    for (int j = 0; j < NLV; ++j)
      *(lds_u4_ptr)(size_t)(vw + j * RV * VROW) = u32x4_t{t.v[j].x, t.v[j].y, t.v[j].z, t.v[j].w};
  }

  // Scores, online softmax and P.V of the tile at tokens t0 .. staged in
  // LDS (ok: its 4-token groups' block bits).
  // kCols: column c also stops at its own key limit lim (the shared
  // chunks of cascade decode, whose columns belong to different rows).
  template <bool kCols>
  __device__ static __forceinline__ void compute(int ok, int t0, int p0, int p1, int lim, float sl, int lane,
                                                 uint32_t lds, State &st) {
    const int g = lane >> 4;
    const int c = lane & 15;
    // S^T = K Q^T: A = K rows (lane: token c, chunk 4 ks + g)
    const uint32_t kr = lds + (uint32_t)(c * KROW + g * 16);
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const bf16x8_t kf = *(lds_b8_ptr)(size_t)(kr + ks * 64);
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, st.qf[ks], s, 0, 0, 0);
    }
    // weights of column c for tokens t0 + 4g .. t0 + 4g + 3
    const bool grp_ok = (ok >> g) & 1;
    float sv[4];
    bool vok[4];
    float cm = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = t0 + 4 * g + r;
      vok[r] = grp_ok && tok >= p0 && tok < p1 && (!kCols || tok < lim);
      sv[r] = vok[r] ? s[r] * sl : -INFINITY;
      cm = fmaxf(cm, sv[r]);
    }
    cm = xor32_max(xor16_max(cm));  // the column's max over the tile
    const bool grow = cm > st.m + kDecodeRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float alpha = grow ? fast_exp2(st.m - cm) : 1.f;  // 0 when m is -inf
      st.m = grow ? cm : st.m;
      st.l *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) st.o[dt] *= alpha;
    }
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = vok[r] ? fast_exp2(sv[r] - st.m) : 0.f;
    st.l += (p[0] + p[1]) + (p[2] + p[3]);
    const uint32_t p01 = pack_bf16x2_rne(p[0], p[1]);
    const uint32_t p23 = pack_bf16x2_rne(p[2], p[3]);
    const v4i16_t pb = __builtin_bit_cast(v4i16_t, make_uint2(p01, p23));
    // O^T += V^T P^T: A = V^T from transposing reads.  In 16-lane group g,
    // lane c sends the address of 4 value dims of one token (token
    // 4g + c / 4, dims 16 dt + 4 (c % 4)) and receives dim 16 dt + c of
    // tokens 4g .. 4g+3.
    const uint32_t vr = lds + (uint32_t)(KBYTES + (4 * g + (c >> 2)) * VROW + (c & 3) * 8);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const v4i16_t vf = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4_ptr)(size_t)(vr + dt * 32));
      st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf, pb, st.o[dt], 0, 0, 0);
    }
  }

  // Q^T fragments of this lane's column from its query row (zero without
  // one), and the empty running state.
  __device__ static __forceinline__ void begin(const uint16_t *qrow, int lane, State &st) {
    const int g = lane >> 4;
    const uint4 *q4 = reinterpret_cast<const uint4 *>(qrow);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const uint4 x = qrow ? q4[4 * ks + g] : make_uint4(0u, 0u, 0u, 0u);
      st.qf[ks] = __builtin_bit_cast(bf16x8_t, x);
    }
    st.m = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) st.o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // Online softmax of kv head kvh's columns over tokens p0 .. p1-1, read
  // through block-table row tab_row; pnew (or -1): the appended token,
  // whose rows are kn, vn (this lane's chunks); with kCols each column
  // stops at its own limit lim.
  template <bool kCols>
  __device__ static __forceinline__ void attend(const DecodeKernelArgs &a, int tab_row, int kvh, int p0, int p1,
                                                int lim, int pnew, uint4 kn, uint4 vn, int lane, uint32_t lds,
                                                State &st) {
    const int tbeg = p0 & ~7;  // tiles start at a multiple of 8
    const int ntiles = p1 > p0 ? (p1 - tbeg + TT - 1) / TT : 0;
    if (ntiles == 0) return;

    const float sl = a.scale_log2;
    Rows w;
    w.tab = read_only(a.block_tables + (size_t)tab_row * a.max_blocks_per_seq);
    w.kbase = static_cast<const char *>(a.k_cache);
    w.vbase = static_cast<const char *>(a.v_cache);
    w.kslot = (size_t)a.num_kv_heads * D * 2;
    w.vslot = (size_t)a.num_kv_heads * DV * 2;
    w.klane = (uint32_t)((size_t)(lane / LK) * w.kslot + (size_t)kvh * D * 2 + (size_t)(lane % LK) * 16);
    w.vlane = (uint32_t)((size_t)(lane / LV) * w.vslot + (size_t)kvh * DV * 2 + (size_t)(lane % LV) * 16);
    // One register set: once a tile is in LDS its registers take the next
    // tile's loads, which are in flight while the staged tile is computed.
    Tile t;
    issue(a, w, tbeg, p1, t);
    for (int i = 0; i < ntiles; ++i) {
      const int t0 = tbeg + i * TT;
      stage(t, t0, p0, p1, pnew, kn, vn, lane, lds);
      const int ok = t.ok;
      if (i + 1 < ntiles) issue(a, w, t0 + TT, p1, t);
      compute<kCols>(ok, t0, p0, p1, lim, sl, lane, lds, st);
    }
  }

  // The wave's totals: the output rows o / l (direct) or the partial
  // (o, m, l) of partition slot `slot`, for the G heads of kv head kvh.
  __device__ static __forceinline__ void write(const DecodeKernelArgs &a, int seq, int kvh, int lane, State &st,
                                               bool direct, int slot) {
    const int g = lane >> 4;
    const int c = lane & 15;
    const float lt = xor32_sum(xor16_sum(st.l));  // the column's sum over the four rows of lanes
    if (c >= G) return;
    const size_t head = (size_t)seq * a.num_heads + (size_t)kvh * G + c;
    if (direct) {
      uint16_t *dst = static_cast<uint16_t *>(a.out) + head * DV + 4 * g;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const f32x4_t v = st.o[dt];
        const float r0 = lt > 0.f ? v[0] / lt : 0.f;
        const float r1 = lt > 0.f ? v[1] / lt : 0.f;
        const float r2 = lt > 0.f ? v[2] / lt : 0.f;
        const float r3 = lt > 0.f ? v[3] / lt : 0.f;
        *reinterpret_cast<uint2 *>(dst + 16 * dt) = make_uint2(pack_bf16x2(r0, r1), pack_bf16x2(r2, r3));
      }
    } else {
      const size_t idx = head * a.max_partitions + slot;
      float *dst = a.ws_o + idx * DV + 4 * g;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const f32x4_t v = st.o[dt];
        *reinterpret_cast<float4 *>(dst + 16 * dt) = make_float4(v[0], v[1], v[2], v[3]);
      }
      if (g == 0) {
        a.ws_m[idx] = st.m;
        a.ws_l[idx] = lt;
      }
    }
  }
};

// One shared chunk of cascade decode for kv head kvh: keys c*chunk ..
// of group g's shared tokens against the columns of column tile ct, column
// j being head j % G of member ct*16/G + j / G of the group.  The keys are
// read through the table of the group's longest row; each column stops at
// its row's own shared tokens (its context may end inside the shared
// part).  Writes partition slot c of every column whose row reads it.
template <int D, int DV, int G>
__device__ __forceinline__ void decode_shared_chunk(const DecodeKernelArgs &a, int grp, int c, int ct, int kvh,
                                                    int lane, uint32_t lds) {
  using K = Bf16DecodeMfma<D, DV, G>;
  static_assert(16 % G == 0, "whole members per column tile");
  const int r0 = a.group_start[grp], r1 = min(a.group_start[grp + 1], a.num_seqs);
  const int mcol = 16 / G;  // members per column tile
  if (ct * mcol >= r1 - r0) return;
  // the group's longest row (lowest index among equals): its table holds
  // every shared block any member reads
  int best = -1, brow = r0;
  for (int i = r0 + lane; i < r1; i += 64) {
    const int cx = decode_context(a, i);
    if (cx > best) {
      best = cx;
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
  const int ctx_max = __builtin_amdgcn_readfirstlane(best);
  const int tab_row = __builtin_amdgcn_readfirstlane(brow);
  const int sh_g = min(a.shared_len[grp], a.shared_cap);
  const int p0 = c * a.shared_chunk;
  const int p1 = min(min(p0 + a.shared_chunk, sh_g), ctx_max);
  if (p1 <= p0) return;  // no row of the group reads this slot

  // this lane's column: member row and head, and the keys it sees
  const int col = lane & 15;
  const int row = r0 + ct * mcol + col / G;
  const bool has_row = row < r1;
  const int lim = has_row ? decode_shared(a, row, decode_context(a, row)) : 0;
  const uint16_t *qrow = has_row ? static_cast<const uint16_t *>(a.q) +
                                       ((size_t)row * a.num_heads + (size_t)kvh * G + col % G) * D
                                 : nullptr;
  typename K::State st;
  K::begin(qrow, lane, st);
  K::template attend<true>(a, tab_row, kvh, p0, p1, lim, -1, make_uint4(0u, 0u, 0u, 0u),
                           make_uint4(0u, 0u, 0u, 0u), lane, lds, st);
  const float lt = xor32_sum(xor16_sum(st.l));
  if (!has_row || p0 >= lim) return;  // the row's reduce does not read slot c
  const int g = lane >> 4;
  const size_t idx = ((size_t)row * a.num_heads + (size_t)kvh * G + col % G) * a.max_partitions + c;
  float *dst = a.ws_o + idx * DV + 4 * g;
#pragma unroll
  for (int dt = 0; dt < K::NDT; ++dt) {
    const f32x4_t v = st.o[dt];
    *reinterpret_cast<float4 *>(dst + 16 * dt) = make_float4(v[0], v[1], v[2], v[3]);
  }
  if (g == 0) {
    a.ws_m[idx] = st.m;
    a.ws_l[idx] = lt;
  }
}

// The partition kernel on Bf16DecodeMfma: work-group (group of 4 kv heads,
// sequence, partition), one wave per kv head; plain decode in size order
// (size_order_item).  Cascade launches number their items z * S + y: the
// groups' shared chunks first (every column tile of every chunk), then each
// row's own tokens after its shared ones in size order (into the slots
// after the row's shared chunks').  The column tiles of one chunk are
// shared_stride items apart, so that (with work-groups dealt round-robin
// to the 8 XCDs by their linear id) they run on one XCD and the chunk's
// K/V rows are fetched into its L2 once.
template <int D, int DV, int G>
__global__ void __launch_bounds__(64 * kDecodeWaves)
// four work-groups per CU (one tile's rows in registers per wave, up to
// 35 KB of LDS per work-group)
__attribute__((amdgpu_waves_per_eu(4)))
decode_partition_mfma_kernel(const DecodeKernelArgs a) {
  using K = Bf16DecodeMfma<D, DV, G>;
  int seq = blockIdx.y;
  int part = blockIdx.z;
  const bool cascade = a.group_start != nullptr;
  // Cascade launches number their items L = z * S + y: the groups' shared
  // chunks first, then the rows' own partitions.  The branch is uniform
  // over the work-group, so every wave meets the barrier below.
  int shared_item = -1, own_item = -1;
  if (cascade) {
    const int L = blockIdx.z * gridDim.y + blockIdx.y;
    if (L < a.shared_items) {
      shared_item = L;
    } else {
      own_item = L - a.shared_items;
      seq = own_item % a.num_seqs;
      part = own_item / a.num_seqs;
    }
  }
  if (shared_item < 0 && a.partition_size > 0 && a.num_seqs <= 64) {
    // (sequence, partition) in size order (for cascade: of the tokens after
    // each row's shared ones)
    __shared__ int s_map[2];
    if (threadIdx.x < 64) {
      int sq = 0, pt = 0;
      const bool ok = size_order_item(a, cascade ? own_item : (int)(blockIdx.z * gridDim.y + blockIdx.y),
                                      threadIdx.x, sq, pt);
      if (threadIdx.x == 0) {
        s_map[0] = ok ? sq : 0;
        s_map[1] = ok ? pt : a.max_partitions;  // no pair: past every sequence's partitions
      }
    }
    __syncthreads();
    seq = __builtin_amdgcn_readfirstlane(s_map[0]);
    part = __builtin_amdgcn_readfirstlane(s_map[1]);
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kvh = blockIdx.x * kDecodeWaves + wave;
  if (kvh >= a.num_kv_heads) return;

  __shared__ __attribute__((aligned(16))) char lds[kDecodeWaves][K::LDS_BYTES];
  typedef __attribute__((address_space(3))) char *lds_char_ptr;
  const uint32_t my_lds = (uint32_t)(size_t)(lds_char_ptr)(&lds[wave][0]);
  if (shared_item >= 0) {
    const int st = a.shared_stride;
    const int ct = (shared_item / st) % a.col_tiles;                    // column tile
    const int pc = (shared_item / (st * a.col_tiles)) * st + shared_item % st;  // (group, chunk)
    if (pc < a.num_groups * a.shared_chunks)
      decode_shared_chunk<D, DV, G>(a, pc / a.shared_chunks, pc % a.shared_chunks, ct, kvh, lane, my_lds);
    return;
  }
  const int ctx = decode_context(a, seq);
  const int sh = decode_shared(a, seq, ctx);
  const int nparts = cascade ? (ctx - sh + a.partition_size - 1) / a.partition_size
                             : decode_num_partitions(a, ctx);
  if (part >= nparts) return;
  const int ps = a.partition_size > 0 ? a.partition_size : ctx;
  const int p0 = sh + part * ps;
  const int p1 = min(ctx, p0 + ps);
  const int slot = cascade ? (sh + a.shared_chunk - 1) / a.shared_chunk + part : part;

  // fused append: the newest token's rows from the input rows
  const bool append = a.new_k != nullptr && !cascade && part == nparts - 1 && ctx > 0;
  const int pnew = append ? ctx - 1 : -1;
  uint4 kn = make_uint4(0u, 0u, 0u, 0u), vn = kn;
  if (append) {
    kn = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.new_k) +
                                          ((size_t)seq * a.num_kv_heads + kvh) * D + (size_t)(lane % K::LK) * 8);
    vn = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.new_v) +
                                          ((size_t)seq * a.num_kv_heads + kvh) * DV + (size_t)(lane % K::LV) * 8);
  }

  typename K::State st;
  const int col = lane & 15;
  K::begin(col < G ? static_cast<const uint16_t *>(a.q) + ((size_t)seq * a.num_heads + (size_t)kvh * G + col) * D
                   : nullptr,
           lane, st);
  K::template attend<false>(a, seq, kvh, p0, p1, p1, pnew, kn, vn, lane, my_lds, st);

  if (append) {
    // the appended rows into the token's slot (after every load of this
    // wave has been consumed); a block outside the pool is skipped
    const int blk = read_only(a.block_tables + (size_t)seq * a.max_blocks_per_seq)[pnew >> a.block_shift];
    if ((unsigned)blk < (unsigned)a.num_blocks) {
      const size_t slot_i = ((size_t)blk << a.block_shift) + (size_t)(pnew & ((1 << a.block_shift) - 1));
      if (lane < K::LK)
        *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(const_cast<void *>(a.k_cache)) +
                                   (slot_i * a.num_kv_heads + kvh) * D + (size_t)lane * 8) = kn;
      if (lane < K::LV)
        *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(const_cast<void *>(a.v_cache)) +
                                   (slot_i * a.num_kv_heads + kvh) * DV + (size_t)lane * 8) = vn;
    }
  }
  K::write(a, seq, kvh, lane, st, !cascade && nparts == 1, slot);
}

// Merge the partitions of every multi-partition sequence:
//   M = max_p m_p,  out = sum_p o_p 2^(m_p - M) / sum_p l_p 2^(m_p - M).
// One work-group of 256 threads per (query head, sequence).  Thread t owns
// four consecutive dimensions (one 16-byte load) of partitions
// p = t / (D/4) (mod 256 / (D/4)), four of them per batch.  The first batch
// is loaded before the context length is known (every slot below
// max_partitions lies inside the workspace; slots past the row's partition
// count are selected out, whatever they hold), so the kernel waits for
// one round trip to memory instead of three.  Each thread merges its
// partitions with a running max (the online-softmax rule); the 256 / (D/4)
// thread groups are then merged through LDS with the same rule.
template <typename T, int D>
__global__ void __launch_bounds__(256)
decode_reduce_kernel(const DecodeKernelArgs a) {
  constexpr int kThreads = 256;
  constexpr int kLanesPerPart = D / 4;               // float4 per lane
  constexpr int kGroups = kThreads / kLanesPerPart;  // partitions per pass
  constexpr int kUnroll = 4;
  constexpr int kBatch = kGroups * kUnroll;          // partitions per batch
  const int head = blockIdx.x;
  const int seq = blockIdx.y;
  const size_t base = ((size_t)seq * a.num_heads + head) * a.max_partitions;
  const int d4 = threadIdx.x % kLanesPerPart;
  const int g = threadIdx.x / kLanesPerPart;
  const float4 *o4 = reinterpret_cast<const float4 *>(a.ws_o);

  float mp[kUnroll], lp[kUnroll];
  float4 op[kUnroll];
  auto load = [&](int p0) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int p = p0 + g + u * kGroups;
      const size_t idx = base + (p < a.max_partitions ? p : 0);
      mp[u] = a.ws_m[idx];
      lp[u] = a.ws_l[idx];
      op[u] = o4[idx * (D / 4) + d4];
    }
  };
  load(0);

  const int ctx = decode_context(a, seq);
  // cascade: a slot per chunk of the shared tokens and per partition of
  // the rest; otherwise one slot per partition, and a single partition was
  // written directly
  const bool cascade = a.group_start != nullptr;
  int nparts = decode_num_partitions(a, ctx);
  if (cascade) {
    const int sh = decode_shared(a, seq, ctx);
    nparts = (sh + a.shared_chunk - 1) / a.shared_chunk + (ctx - sh + a.partition_size - 1) / a.partition_size;
  }
  if (!cascade && nparts <= 1) return;
  // (a cascade row of context 0 has no slot: its output is zero)

  // this thread's running (m, l, o) over its partitions; a partition with
  // no token has m = -inf and weight 0
  float m = -INFINITY, l = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int p0 = 0; p0 < nparts; p0 += kBatch) {
    if (p0 > 0) load(p0);
    float bm = -INFINITY;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const bool in = p0 + g + u * kGroups < nparts;
      mp[u] = in ? mp[u] : -INFINITY;
      lp[u] = in ? lp[u] : 0.f;
      op[u] = in ? op[u] : make_float4(0.f, 0.f, 0.f, 0.f);
      bm = fmaxf(bm, mp[u]);
    }
    if (bm == -INFINITY) continue;
    const float mn = fmaxf(m, bm);
    const float alpha = fast_exp2(m - mn);  // 0 while m is still -inf
    o.x *= alpha;
    o.y *= alpha;
    o.z *= alpha;
    o.w *= alpha;
    l *= alpha;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float f = (mp[u] == -INFINITY) ? 0.f : fast_exp2(mp[u] - mn);
      o.x = fmaf(op[u].x, f, o.x);
      o.y = fmaf(op[u].y, f, o.y);
      o.z = fmaf(op[u].z, f, o.z);
      o.w = fmaf(op[u].w, f, o.w);
      l = fmaf(lp[u], f, l);
    }
    m = mn;
  }

  __shared__ float4 sm_o[kGroups][kLanesPerPart];
  __shared__ float sm_m[kGroups], sm_l[kGroups];
  sm_o[g][d4] = o;
  if (d4 == 0) {
    sm_m[g] = m;
    sm_l[g] = l;
  }
  __syncthreads();
  if (g == 0) {
    float M = sm_m[0];
#pragma unroll
    for (int i = 1; i < kGroups; ++i) M = fmaxf(M, sm_m[i]);
    float4 ot = make_float4(0.f, 0.f, 0.f, 0.f);
    float lt = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int i = 0; i < kGroups; ++i) {
        const float mi = sm_m[i];
        const float f = (mi == -INFINITY) ? 0.f : fast_exp2(mi - M);
        const float4 v = sm_o[i][d4];
        ot.x = fmaf(v.x, f, ot.x);
        ot.y = fmaf(v.y, f, ot.y);
        ot.z = fmaf(v.z, f, ot.z);
        ot.w = fmaf(v.w, f, ot.w);
        lt = fmaf(sm_l[i], f, lt);
      }
    }
    const size_t ob = ((size_t)seq * a.num_heads + head) * D + d4 * 4;
    store_one<T>(a.out, ob + 0, lt > 0.f ? ot.x / lt : 0.f);
    store_one<T>(a.out, ob + 1, lt > 0.f ? ot.y / lt : 0.f);
    store_one<T>(a.out, ob + 2, lt > 0.f ? ot.z / lt : 0.f);
    store_one<T>(a.out, ob + 3, lt > 0.f ? ot.w / lt : 0.f);
  }
}

// ---------------------------------------------------------------- host
static DecodeKernelArgs make_kernel_args(const DecodeArgs &a) {
  DecodeKernelArgs k;
  k.out = a.out;
  k.q = a.q;
  k.k_cache = a.cache.k;
  k.v_cache = a.cache.v;
  k.block_tables = a.block_tables;
  k.context_lens = a.context_lens;
  k.ws_m = a.ws_m;
  k.ws_l = a.ws_l;
  k.ws_o = a.ws_o;
  k.num_heads = a.num_heads;
  k.num_kv_heads = a.cache.num_kv_heads;
  k.num_blocks = a.cache.num_blocks;
  int shift = 0;
  while ((1 << shift) < a.cache.block_size) ++shift;
  k.block_shift = shift;
  k.max_blocks_per_seq = a.max_blocks_per_seq;
  const int64_t table_cap = (int64_t)a.max_blocks_per_seq * a.cache.block_size;
  k.ctx_cap = (int)(table_cap < a.max_context_len ? table_cap : a.max_context_len);
  k.partition_size = a.partition_size;
  k.max_partitions = a.max_partitions;
  k.num_seqs = a.num_seqs;
  k.scale_log2 = a.scale * kLog2e;
  k.group_start = a.group_start;
  k.shared_len = a.shared_len;
  k.num_groups = a.num_groups;
  k.shared_chunk = a.shared_chunk;
  k.shared_cap = a.shared_cap;
  k.shared_chunks = a.shared_chunks;
  k.shared_items = 0;
  k.shared_stride = 1;
  k.col_tiles = 1;
  k.query_start_loc = a.query_start_loc;
  k.num_prefill_seqs = a.num_prefill_seqs;
  k.new_k = a.new_k;
  k.new_v = a.new_v;
  return k;
}

// own-token partitions a cascade row may have: its tokens after the
// shared ones, at most the (clamped) context
int cascade_own_partitions(const DecodeArgs &a) {
  const int64_t table_cap = (int64_t)a.max_blocks_per_seq * a.cache.block_size;
  const int64_t cap = table_cap < a.max_context_len ? table_cap : a.max_context_len;
  const int64_t n = (cap + a.partition_size - 1) / a.partition_size;
  return (int)(n > 1 ? n : 1);
}

// Launch items of a cascade's shared chunks: (group, chunk) pairs in runs
// of `stride`, each run repeated for every column tile, so that the column
// tiles of one chunk are `stride` items apart.  With gridDim.x work-groups
// per item and linear work-group ids dealt round-robin over 8 XCDs, items
// 8 / gcd(gridDim.x, 8) apart run on the same XCD.
int64_t cascade_shared_items(const DecodeArgs &a, int col_tiles, int &stride) {
  const int x = (a.cache.num_kv_heads + kDecodeWaves - 1) / kDecodeWaves;
  stride = (x % 8 == 0) ? 1 : (x % 4 == 0) ? 2 : (x % 2 == 0) ? 4 : 8;
  const int64_t pairs = (int64_t)a.num_groups * a.shared_chunks;
  return (pairs + stride - 1) / stride * stride * col_tiles;
}

int cascade_grid_z(const DecodeArgs &a, int col_tiles) {
  int stride;
  const int64_t items = cascade_shared_items(a, col_tiles, stride) + (int64_t)a.num_seqs * cascade_own_partitions(a);
  const int64_t z = (items + a.num_seqs - 1) / a.num_seqs;
  return (int)(z < 0x7fffffff ? z : 0x7fffffff);
}

template <typename T, int D, int DV, int G>
static hipError_t launch_partition_t(const DecodeArgs &a, hipStream_t stream) {
  DecodeKernelArgs k = make_kernel_args(a);
  dim3 grid(a.max_partitions, a.cache.num_kv_heads, a.num_seqs);
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (a.query_start_loc) return hipErrorNotSupported;  // prefill rows run on the generic kernel only
    // every bf16 decode (plain and cascade, any head dim pair) on the
    // matrix-core kernel; a cascade launch also runs the groups' shared
    // chunks, ahead of the rows' own tokens in the grid
    int zs = a.max_partitions;
    if (a.group_start) {
      k.col_tiles = (a.max_group_size * G + 15) / 16;
      k.shared_items = (int)cascade_shared_items(a, k.col_tiles, k.shared_stride);
      zs = cascade_grid_z(a, k.col_tiles);
    }
    grid = dim3((a.cache.num_kv_heads + kDecodeWaves - 1) / kDecodeWaves, a.num_seqs, zs);
    hipLaunchKernelGGL((decode_partition_mfma_kernel<D, DV, G>), grid, dim3(64 * kDecodeWaves), 0, stream, k);
  } else {
    // (cascade launches are bf16: never here)
    hipLaunchKernelGGL((decode_partition_kernel<T, D, DV, G>), grid, dim3(DecodeShape<T, D>::kThreads), 0,
                       stream, k);
  }
  return hipGetLastError();
}

template <typename T, int D, int DV>
static hipError_t launch_partition_g(const DecodeArgs &a, hipStream_t stream) {
  switch (a.num_heads / a.cache.num_kv_heads) {
    case 1: return launch_partition_t<T, D, DV, 1>(a, stream);
    case 2: return launch_partition_t<T, D, DV, 2>(a, stream);
    case 4: return launch_partition_t<T, D, DV, 4>(a, stream);
    case 8: return launch_partition_t<T, D, DV, 8>(a, stream);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t launch_partition_d(const DecodeArgs &a, hipStream_t stream) {
  const int dk = a.cache.head_dim, dv = a.cache.head_dim_v;
  if (dk == 64 && dv == 64) return launch_partition_g<T, 64, 64>(a, stream);
  if (dk == 128 && dv == 128) return launch_partition_g<T, 128, 128>(a, stream);
  if (dk == 128 && dv == 64) return launch_partition_g<T, 128, 64>(a, stream);
  if (dk == 64 && dv == 128) return launch_partition_g<T, 64, 128>(a, stream);
  return hipErrorInvalidValue;
}

bool decode_fast_path(const DecodeArgs &a) {
  const int g = a.cache.num_kv_heads > 0 ? a.num_heads / a.cache.num_kv_heads : 0;
  return a.cache.dtype == 1 && g >= 1 && g <= 8 &&
         !a.query_start_loc;
}

hipError_t launch_decode_partition(const DecodeArgs &a, hipStream_t stream) {
  if (a.new_k && !decode_fast_path(a)) return hipErrorInvalidValue;  // the ABI routes these to the plain write
  if (a.num_seqs == 0) return hipSuccess;
  if (a.cache.dtype == 1) return launch_partition_d<bf16_t>(a, stream);
  return launch_partition_d<float>(a, stream);
}

template <typename T, int D>
static hipError_t launch_reduce_t(const DecodeArgs &a, hipStream_t stream) {
  const DecodeKernelArgs k = make_kernel_args(a);
  dim3 grid(a.num_heads, a.num_seqs);
  hipLaunchKernelGGL((decode_reduce_kernel<T, D>), grid, dim3(256), 0, stream, k);
  return hipGetLastError();
}

hipError_t launch_decode_reduce(const DecodeArgs &a, hipStream_t stream) {
  if (a.num_seqs == 0 || a.partition_size <= 0 || a.max_partitions <= 1) return hipSuccess;
  const bool bf = (a.cache.dtype == 1);
  switch (a.cache.head_dim_v) {  // the width of the partials and output rows
    case 64: return bf ? launch_reduce_t<bf16_t, 64>(a, stream) : launch_reduce_t<float, 64>(a, stream);
    case 128: return bf ? launch_reduce_t<bf16_t, 128>(a, stream) : launch_reduce_t<float, 128>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
