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
// How it maps to gfx950:
//  * One work-group (4 waves) per (partition, kv head, sequence).  It owns
//    the G = num_heads / num_kv_heads query heads of that kv head, so each
//    K/V byte of the partition is read from HBM exactly once for all G
//    heads.
//  * One token's K row for one kv head is head_dim contiguous elements
//    (256 B for bf16 x 128), read by L = row_bytes / 16 lanes with one
//    128-bit load each.  A wave covers 64 / L tokens per load instruction
//    and keeps kUnroll loads of K and kUnroll loads of V in flight per
//    lane.
//  * The q.k partial sums are reduced across the L lanes of a row with DPP
//    (quad permutes and row rotates), so no LDS traffic is needed.
//  * Each wave runs its own online softmax over its chunks (running max m,
//    running sum l, accumulator rescaled by 2^(m_old - m_new)).  Scores are
//    kept in base-2 units: q is pre-multiplied by scale * log2(e), so that
//    one v_exp_f32 gives each weight.  A token outside the context or in an
//    invalid block is *selected out*: its score is -inf, its weight is
//    exactly 0, and its V is never loaded, so stale or NaN pool contents
//    cannot leak in.
//  * The four waves merge (m, l, o) through LDS with the same rescaling
//    rule.  A sequence that fits in one partition is normalised and stored
//    directly.  Otherwise the partition's (m, l, o) go to the workspace and
//    the reduce kernel merges the partitions.
//  * The block id of each load is the same for the whole wave (a load
//    covers 64 / L consecutive tokens inside one block), so block-table
//    reads are scalar loads.
//  * Key and value head dims may differ (section 4.1 of the same page):
//    the L lanes of a token's K row also cover its V row, each lane
//    loading DV / L elements of V (8, 16 or 32 bytes), so the softmax
//    weights of a lane's token serve both.
//  * For key head dim 128 the bf16 path takes the rows of a load across kv
//    heads instead of tokens (Bf16DecodeRows): a work-group covers 4 kv
//    heads, and each load instruction reads one token's rows of those 4
//    heads, 1 KB contiguous, instead of 256-byte slices at the 2 KB token
//    stride.  Long and uniform contexts read 3-6% faster this way.  Each
//    wave keeps its next step's K and V loads in flight while it computes
//    the current step (two register sets), and the four waves' totals are
//    merged in a tree through two LDS slots, which keeps the staging of
//    eight query heads per kv head at 33 KB (three work-groups per CU).
//    It serves separate value head dims and the own-token pass of cascade
//    decode.
//  * Plain bf16 decode with key and value head dims 128 runs on the matrix
//    cores instead (Bf16DecodeMfma, below): per kv head, the scores of 16
//    tokens and their weighted V rows are two small MFMA products, so the
//    vector work per token no longer grows with the query heads per kv
//    head.
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
  int shared_cap;        // shared tokens are clamped to this (the chunks launched)
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
// bf16 fast path (G in {1, 2, 4, 8}, equal key and value head dims).  Same
// decomposition as the generic kernel above, with the per-token work cut
// down for the VALU:
//  * q.k in bf16 pairs with v_dot2_f32_bf16 (products exact, fp32 sums), no
//    widening of K;
//  * a reduce-scatter across the row instead of an all-reduce: after it,
//    lane c of a row holds the full score of head c % G only, so each lane
//    computes one exponential per token;
//  * P.V in bf16 pairs over two tokens: a lane rounds its head's weights of
//    tokens t and t+1 to bf16 (nearest even) and packs them, every lane of
//    the row takes each head's packed pair from its owner with DPP moves, V
//    elements of the two tokens are interleaved with v_perm_b32, and
//    v_dot2_f32_bf16 adds both products to the fp32 accumulator.  The
//    running sum l uses the fp32 weights;
//  * the running max is a reference, moved only when a chunk exceeds it by
//    more than 2^8 (the rescale of l and the accumulators is then rare);
//    exact in real arithmetic, like the eager rescale;
//  * the K and V loads of a wave's next chunk are issued as soon as the
//    registers of the current chunk are consumed, so they overlap the
//    softmax and P.V work of the current chunk.
constexpr int kDecodeUnroll = 8;      // tokens per wave step
constexpr int kDecodeUnrollWide = 4;  // more than 32 accumulators per lane: fewer loads in flight, fewer registers
constexpr int kDecodeWaves = 4;       // waves per work-group
constexpr int kRowsUnroll = 4;        // the same for the row-layout kernel, which pipelines two steps
constexpr int kRowsUnrollWide = 2;
// Grid order of the partition kernels: kv head fastest, then the
// (sequence, partition) pairs by size: every full partition first, then the
// partial last partitions, longest first, so that the work-groups
// dispatched last are the short ones (batches of at most 64 sequences;
// larger ones, and cascade launches, take sequence then partition, so that
// the partitions that exist for every sequence are dispatched first and
// the empty ones past short contexts come last).

// Reduce-scatter of G per-lane partial sums over a row of L lanes.  Slot j
// of lane c holds the partial sum of head j ^ (c % G) (the query heads are
// loaded in that lane-dependent order), so at every exchange the partner
// lane holds the head a lane keeps in a fixed slot and no selects are
// needed.  Lane c returns the row total of head c % G (all lanes of the row
// with the same c % G get the same value).
template <int L, int G>
__device__ __forceinline__ float row_scatter_sum(const float (&v)[G]) {
  float r;
  if constexpr (G == 8) {
    // the half-row mirror pairs lane c with lane c ^ 7, whose slot 7 - j
    // holds the head of slot j here; then xor 2 and xor 1.  The three
    // partners generate all eight lanes of the group.
    float x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = v[j] + dpp_f32<kDppRowHalfMirror>(v[7 - j]);
    const float y0 = x[0] + dpp_f32<kDppQuadXor2>(x[2]);
    const float y1 = x[1] + dpp_f32<kDppQuadXor2>(x[3]);
    r = y0 + dpp_f32<kDppQuadXor1>(y1);
  } else if constexpr (G == 4) {
    const float x0 = v[0] + dpp_f32<kDppQuadXor1>(v[1]);
    const float x2 = v[2] + dpp_f32<kDppQuadXor1>(v[3]);
    r = x0 + dpp_f32<kDppQuadXor2>(x2);
  } else if constexpr (G == 2) {
    r = v[0] + dpp_f32<kDppQuadXor1>(v[1]);
    r += dpp_f32<kDppQuadXor2>(r);
  } else {
    r = v[0];
    r += dpp_f32<kDppQuadXor1>(r);
    r += dpp_f32<kDppQuadXor2>(r);
  }
  // the rest of the row: the other quads (G <= 4) or the other 8-lane
  // group of a 16-lane row (G = 8)
  if constexpr (L == 16) {
    if constexpr (G < 8) r += dpp_f32<kDppRowRor4>(r);
    r += dpp_f32<kDppRowRor8>(r);
  } else {
    static_assert(L == 8, "rows of 8 or 16 lanes");
    if constexpr (G < 8) r += swizzle_xor4(r);
  }
  return r;
}

// max / sum of a value over the rows of a wave (lanes c, c+L, c+2L, ...)
template <int L>
__device__ __forceinline__ float rows_max(float x) {
  if constexpr (L == 8) x = fmaxf(x, dpp_f32<kDppRowRor8>(x));
  x = xor16_max(x);
  return xor32_max(x);
}
template <int L>
__device__ __forceinline__ float rows_sum(float x) {
  if constexpr (L == 8) x += dpp_f32<kDppRowRor8>(x);
  x = xor16_sum(x);
  return xor32_sum(x);
}

// value of head H for this lane's row, from the lane of the row that owns
// it (lane c owns head c % G; col = lane % L)
template <int G, int H>
__device__ __forceinline__ uint32_t from_head(uint32_t x, int col) {
  if constexpr (G == 1) {
    return x;
  } else if constexpr (G <= 4) {
    return quad_bcast<H>(x);
  } else {
    // quads of parity j hold heads 4j .. 4j+3: quad lane H % 4 has head H
    // in the quads of parity H / 4, and the half-row mirror brings it to
    // the quads of the other parity
    const uint32_t q = quad_bcast<H % 4>(x);
    const uint32_t o = dpp_u32<kDppRowHalfMirror>(q);
    return (((col >> 2) & 1) == (H >> 2)) ? q : o;
  }
}
// out[h] = the value of head h, for every head of the group
template <int G, int H = 0>
__device__ __forceinline__ void every_head(uint32_t x, int col, uint32_t (&out)[G]) {
  if constexpr (H < G) {
    out[H] = from_head<G, H>(x, col);
    every_head<G, H + 1>(x, col, out);
  }
}
template <int G>
__device__ __forceinline__ void every_head(float x, int col, float (&out)[G]) {
  uint32_t u[G];
  every_head<G>(__float_as_uint(x), col, u);
#pragma unroll
  for (int h = 0; h < G; ++h) out[h] = __uint_as_float(u[h]);
}

// A wave rescales its running sums only when a head's max grows by more
// than this many base-2 units; until then the weights exp2(s - m) may reach
// 2^8, which the fp32 sums and the bf16 weights hold exactly as well.
constexpr float kDecodeRescaleSlack = 8.f;

// Addressing of one wave step.  Load u of chunk c covers the R tokens
// tok0 .. tok0+R-1 (tok0 = chunk start + u*R), all in one block, so the
// block id and the element offset of that token group are the same for the
// whole wave and live in scalar registers.  A lane adds its own fixed byte
// offset (its row times the slot stride plus its 16-byte column).
// Read-only view for inputs that no work-group writes during a launch
// (block tables, context lengths): loads through the constant address
// space stay scalar for wave-uniform indices even after the kernel's own
// stores and fences.
typedef const __attribute__((address_space(4))) int32_t *ro_i32_ptr;
__device__ __forceinline__ ro_i32_ptr read_only(const int32_t *p) { return (ro_i32_ptr)(p); }

template <int U, int R>
__device__ __forceinline__ void chunk_rows(size_t (&off)[U], bool (&ok)[U], const int32_t *bt, int cbase,
                                           int p1, int shift, int bs_mask, int num_blocks,
                                           size_t slot_stride, int max_blocks) {
  // table reads are unconditional (index clamped into the row) so that all
  // of them are in flight together
  const ro_i32_ptr tab = read_only(bt);
  int blk[U];
#pragma unroll
  for (int u = 0; u < U; ++u) blk[u] = tab[min((cbase + u * R) >> shift, max_blocks - 1)];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int tok0 = cbase + u * R;
    ok[u] = (tok0 < p1) && ((unsigned)blk[u] < (unsigned)num_blocks);
    // selects on the inputs, not on the product, keep this branch-free so
    // that the table reads are not serialised by waits before branches
    const uint32_t b = ok[u] ? (uint32_t)blk[u] : 0u;
    const uint32_t t = ok[u] ? (uint32_t)(tok0 & bs_mask) : 0u;
    off[u] = (((size_t)b << shift) + t) * slot_stride;  // 0: pool start
  }
}

// Unconditional loads: a lane past the context still reads inside the
// pool (its own row of the same block, or the first row of the pool when
// the block id is invalid), and its values are discarded by selects.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

template <int U>
__device__ __forceinline__ void chunk_load(uint4 (&buf)[U], const size_t (&off)[U], const uint16_t *base,
                                           uint32_t lane_bytes) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const char *ptr = reinterpret_cast<const char *>(base + off[u]) + lane_bytes;
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(ptr));
    buf[u] = make_uint4(v.x, v.y, v.z, v.w);
  }
}

// The same for a V slice of VW words (8, 16 or 32 bytes) per lane.
template <int U, int VW>
__device__ __forceinline__ void chunk_load_words(uint32_t (&buf)[U][VW], const size_t (&off)[U],
                                                 const uint16_t *base, uint32_t lane_bytes) {
  typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const char *ptr = reinterpret_cast<const char *>(base + off[u]) + lane_bytes;
    if constexpr (VW == 2) {
      const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t *>(ptr));
      buf[u][0] = v.x, buf[u][1] = v.y;
    } else {
#pragma unroll
      for (int i = 0; i < VW / 4; ++i) {
        const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(ptr) + i);
        buf[u][4 * i] = v.x, buf[u][4 * i + 1] = v.y, buf[u][4 * i + 2] = v.z, buf[u][4 * i + 3] = v.w;
      }
    }
  }
}

// Per-wave online softmax of the G query heads of kv head `kvh` over the
// tokens p0 .. p1-1 of sequence `seq`.  The wave takes chunks of CH tokens
// c = wave, wave + W, ...; on return m (base-2 units) and l hold the wave's
// running max and sum of head col % G, acc the wave's P.V sums (rows already
// summed, valid in every lane).  D is the key head dim, DV the value head
// dim: the L lanes that read a token's K row (16 bytes each) also read its
// V row, EV = DV / L elements each (8, 16 or 32 bytes).
template <int D, int DV, int G>
struct Bf16Decode {
  static constexpr int L = D / 8;   // lanes per token row (8 bf16 of K per lane)
  static constexpr int R = 64 / L;  // token rows per load instruction
  static constexpr int EV = DV / L; // V elements per lane
  static constexpr int VW = EV / 2; // V words (bf16 pairs) per lane
  static constexpr int U = (G * EV > 32) ? kDecodeUnrollWide : kDecodeUnroll;
  static constexpr int CH = R * U;  // tokens per wave step
  static constexpr int W = kDecodeWaves;
  static_assert(U % 2 == 0, "tokens are paired for the P.V dot products");
  static_assert(VW == 2 || VW == 4 || VW == 8, "8, 16 or 32 bytes of V per lane");

  __device__ static __forceinline__ void attend(const DecodeKernelArgs &a, int seq, int kvh, int p0, int p1,
                                                int wave, int lane, float &m, float &l, float (&acc)[G][EV]) {
    const int row = lane / L;
    const int col = lane % L;
    uint32_t qp[G][4];
    {
      const uint4 *qv = reinterpret_cast<const uint4 *>(
          static_cast<const uint16_t *>(a.q) + ((size_t)seq * a.num_heads + (size_t)kvh * G) * D);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const uint4 c = qv[(h ^ (col & (G - 1))) * L + col];  // slot h: head h ^ (col % G)
        qp[h][0] = c.x;
        qp[h][1] = c.y;
        qp[h][2] = c.z;
        qp[h][3] = c.w;
      }
    }
    const float sl = a.scale_log2;
    const size_t slot_stride = (size_t)a.num_kv_heads * D;
    const uint16_t *kbase = static_cast<const uint16_t *>(a.k_cache) + (size_t)kvh * D;
    const uint16_t *vbase = static_cast<const uint16_t *>(a.v_cache) + (size_t)kvh * DV;
    const uint32_t lane_bytes = (uint32_t)(((size_t)row * slot_stride + (size_t)col * 8) * 2);
    const uint32_t vlane_bytes = (uint32_t)(((size_t)row * a.num_kv_heads * DV + (size_t)col * EV) * 2);
    const int32_t *bt = a.block_tables + (size_t)seq * a.max_blocks_per_seq;
    const int shift = a.block_shift;
    const int bs_mask = (1 << shift) - 1;

    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EV; ++e) acc[h][e] = 0.f;

    const int ntok = p1 - p0;
    const int nchunks = ntok > 0 ? (ntok + CH - 1) / CH : 0;
    for (int c = wave; c < nchunks; c += W) {
      const int cbase = p0 + c * CH;
      size_t off[U];
      bool ok[U];
      chunk_rows<U, R>(off, ok, bt, cbase, p1, shift, bs_mask, a.num_blocks, slot_stride,
                       a.max_blocks_per_seq);
      uint4 kr[U];
      uint32_t vr[U][VW];
      chunk_load<U>(kr, off, kbase, lane_bytes);
      if constexpr (DV == D) {
        uint4 v4[U];
        chunk_load<U>(v4, off, vbase, lane_bytes);
#pragma unroll
        for (int u = 0; u < U; ++u) vr[u][0] = v4[u].x, vr[u][1] = v4[u].y, vr[u][2] = v4[u].z, vr[u][3] = v4[u].w;
      } else {
        // V's slot stride is DV / D times K's: the same slot, scaled offset
        size_t voff[U];
#pragma unroll
        for (int u = 0; u < U; ++u) voff[u] = (DV > D) ? off[u] << 1 : off[u] >> 1;
        chunk_load_words<U, VW>(vr, voff, vbase, vlane_bytes);
      }
      bool valid[U];
#pragma unroll
      for (int u = 0; u < U; ++u) valid[u] = ok[u] && (cbase + u * R + row < p1);

      float s[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float d[G];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float t = dot2_bf16(qp[h][0], kr[u].x, 0.f);
          t = dot2_bf16(qp[h][1], kr[u].y, t);
          t = dot2_bf16(qp[h][2], kr[u].z, t);
          d[h] = dot2_bf16(qp[h][3], kr[u].w, t);
        }
        const float r = row_scatter_sum<L, G>(d);
        s[u] = valid[u] ? r * sl : -INFINITY;
      }
      float cm = s[0];
#pragma unroll
      for (int u = 1; u < U; ++u) cm = fmaxf(cm, s[u]);
      cm = rows_max<L>(cm);
      // lazy rescale: a head's reference max moves only when the chunk
      // exceeds it by more than the slack (always on its first valid chunk,
      // when m is still -inf)
      const bool grow = cm > m + kDecodeRescaleSlack;
      if (__builtin_amdgcn_ballot_w64(grow)) {
        const float alpha = grow ? fast_exp2(m - cm) : 1.f;  // 0 when m is -inf
        m = grow ? cm : m;
        l *= alpha;
        float ah[G];
        every_head<G>(alpha, col, ah);
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < EV; ++e) acc[h][e] *= ah[h];
      }
      float p[U];
      float psum = 0.f;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        p[u] = valid[u] ? fast_exp2(s[u] - m) : 0.f;
        psum += p[u];
      }
      l += psum;

      // rows outside the context (or in an invalid block) may hold anything,
      // NaN included: select them to zero so that weight 0 gives exactly 0
      bool full = cbase + CH <= p1;
#pragma unroll
      for (int u = 0; u < U; ++u) full = full && ok[u];
      if (!full) {
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (!valid[u]) {
#pragma unroll
            for (int j = 0; j < VW; ++j) vr[u][j] = 0;
          }
      }
#pragma unroll
      for (int u = 0; u < U; u += 2) {
        // element 2j (2j+1) of the two tokens in one bf16 pair
        uint32_t vp[EV];
#pragma unroll
        for (int j = 0; j < VW; ++j) {
          vp[2 * j] = interleave_lo(vr[u][j], vr[u + 1][j]);
          vp[2 * j + 1] = interleave_hi(vr[u][j], vr[u + 1][j]);
        }
        // this lane's head's two weights, rounded to bf16 and packed, then
        // the packed pair of every head from the lane that owns it
        uint32_t pk[G];
        every_head<G>(pack_bf16x2_rne(p[u], p[u + 1]), col, pk);
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < EV; ++e) acc[h][e] = dot2_bf16(pk[h], vp[e], acc[h][e]);
      }
    }

    // wave totals: sum the rows
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EV; ++e) acc[h][e] = rows_sum<L>(acc[h][e]);
    l = rows_sum<L>(l);
  }

  // Adds the newest token of sequence `seq` (position pos), whose K and V
  // rows come from the fused-append input instead of the cache, to a wave's
  // totals (m, l, acc) as attend returns them, and writes the rows into the
  // token's cache slot.  Every row of lanes takes the same token, so the
  // totals stay the same in every row.  The weight is rounded to bf16 before
  // it multiplies V and the sum takes it unrounded, as in attend.  A token
  // whose block id is outside the pool is left out and not written, as the
  // separate cache write and the partition loop would leave it.
  __device__ static __forceinline__ void attend_new(const DecodeKernelArgs &a, int seq, int kvh, int pos,
                                                    int lane, float &m, float &l, float (&acc)[G][EV]) {
    const int col = lane % L;
    const int blk = read_only(a.block_tables + (size_t)seq * a.max_blocks_per_seq)[pos >> a.block_shift];
    if ((unsigned)blk >= (unsigned)a.num_blocks) return;
    const size_t in_row = ((size_t)seq * a.num_kv_heads + kvh) * D + (size_t)col * 8;
    const size_t in_vrow = ((size_t)seq * a.num_kv_heads + kvh) * DV + (size_t)col * EV;
    const uint4 kc = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.new_k) + in_row);
    Vec<bf16_t, EV> vc;
    vc.load(static_cast<const bf16_t *>(a.new_v) + in_vrow);
    const uint4 *qv = reinterpret_cast<const uint4 *>(
        static_cast<const uint16_t *>(a.q) + ((size_t)seq * a.num_heads + (size_t)kvh * G) * D);
    float d[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const uint4 qc = qv[(h ^ (col & (G - 1))) * L + col];  // slot h: head h ^ (col % G)
      float t = dot2_bf16(qc.x, kc.x, 0.f);
      t = dot2_bf16(qc.y, kc.y, t);
      t = dot2_bf16(qc.z, kc.z, t);
      d[h] = dot2_bf16(qc.w, kc.w, t);
    }
    const float s = row_scatter_sum<L, G>(d) * a.scale_log2;  // head col % G
    const float m_new = fmaxf(m, s);
    const float alpha = fast_exp2(m - m_new);  // 0 while m is still -inf
    const float p = fast_exp2(s - m_new);
    m = m_new;
    l = l * alpha + p;
    float vf[EV];
    vc.widen(vf);
    float ah[G], pb[G];
    every_head<G>(alpha, col, ah);
    every_head<G>(p, col, pb);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float pr = bf16_lo(pack_bf16x2_rne(pb[h], 0.f));  // the weight rounded to bf16
#pragma unroll
      for (int e = 0; e < EV; ++e) acc[h][e] = fmaf(pr, vf[e], acc[h][e] * ah[h]);
    }
    if (lane < L) {
      const size_t slot = ((size_t)blk << a.block_shift) + (size_t)(pos & ((1 << a.block_shift) - 1));
      const size_t at = slot * a.num_kv_heads * D + (size_t)kvh * D + (size_t)col * 8;
      const size_t vat = slot * a.num_kv_heads * DV + (size_t)kvh * DV + (size_t)col * EV;
      *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(const_cast<void *>(a.k_cache)) + at) = kc;
      uint32_t *vdst = reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(const_cast<void *>(a.v_cache)) + vat);
      if constexpr (VW == 2) {
        *reinterpret_cast<uint2 *>(vdst) = make_uint2(vc.w[0], vc.w[1]);
      } else {
#pragma unroll
        for (int i = 0; i < VW / 4; ++i)
          reinterpret_cast<uint4 *>(vdst)[i] = make_uint4(vc.w[4 * i], vc.w[4 * i + 1], vc.w[4 * i + 2], vc.w[4 * i + 3]);
      }
    }
  }

  // LDS staging of the W waves' (m, l, acc) for the combine
  struct Stage {
    float m[W][G];
    float l[W][G];
    float o[W][G][DV];
  };

  __device__ static __forceinline__ void stage(Stage &sm, int wave, int lane, float m, float l,
                                               const float (&acc)[G][EV]) {
    const int col = lane % L;
    if (lane < L) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EV; ++e) sm.o[wave][h][col * EV + e] = acc[h][e];
    }
    if (lane < G) {  // lane c of row 0 owns head c
      sm.m[wave][lane] = m;
      sm.l[wave][lane] = l;
    }
  }

  // combine of output i = h * DV + d over the staged waves: M = max, o and
  // the sum scaled to M (both 0 when every wave is empty)
  __device__ static __forceinline__ void combine(const Stage &sm, int i, float &M, float &o, float &lt) {
    const int h = i / DV;
    const int d = i - h * DV;
    M = sm.m[0][h];
#pragma unroll
    for (int w = 1; w < W; ++w) M = fmaxf(M, sm.m[w][h]);
    o = 0.f;
    lt = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float mw = sm.m[w][h];
        const float f = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
        o = fmaf(sm.o[w][h][d], f, o);
        lt = fmaf(sm.l[w][h], f, lt);
      }
    }
  }
};

// The same decode with the rows of one load instruction taken across kv
// heads instead of tokens: the R = 64 / L rows of a load are one token's K
// (or V) rows for kv heads kvh0 .. kvh0+R-1, which lie next to each other in
// the pool (R * 256 bytes contiguous for head dim 128), and a wave step takes
// U consecutive tokens.  A work-group then covers R kv heads of a partition
// and reads whole contiguous stretches of each token's row instead of one
// head's 256-byte slice at the row stride.  Every lane keeps one kv head
// (its row) for all its tokens: no sums across the rows of a wave, and the
// validity of a token is the same for the whole wave.
template <int D, int DV, int G>
struct Bf16DecodeRows {
  static constexpr int L = D / 8;   // lanes per row (8 bf16 of K per lane)
  static constexpr int R = 64 / L;  // kv heads per load instruction
  static constexpr int EV = DV / L; // V elements per lane
  static constexpr int VW = EV / 2; // V words (bf16 pairs) per lane
  // tokens per wave step (two steps' rows are held at once)
  static constexpr int U = (G * EV > 32) ? kRowsUnrollWide : kRowsUnroll;
  static constexpr int W = kDecodeWaves;
  static_assert(U % 2 == 0, "tokens are paired for the P.V dot products");
  static_assert(VW == 2 || VW == 4 || VW == 8, "8, 16 or 32 bytes of V per lane");

  // This lane's kv head: kvh0 + its row, or kvh0 for a row past the last
  // kv head (such a row reads kv head kvh0 and its results are dropped).
  __device__ static __forceinline__ int lane_head(const DecodeKernelArgs &a, int kvh0, int lane) {
    const int kvh = kvh0 + lane / L;
    return kvh < a.num_kv_heads ? kvh : kvh0;
  }

  __device__ static __forceinline__ void attend(const DecodeKernelArgs &a, int seq, int kvh0, int p0, int p1,
                                                int wave, int lane, float &m, float &l, float (&acc)[G][EV]) {
    const int col = lane % L;
    const int kvh = lane_head(a, kvh0, lane);
    uint32_t qp[G][4];
    {
      const uint4 *qv = reinterpret_cast<const uint4 *>(
          static_cast<const uint16_t *>(a.q) + ((size_t)seq * a.num_heads + (size_t)kvh * G) * D);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const uint4 c = qv[(h ^ (col & (G - 1))) * L + col];  // slot h: head h ^ (col % G)
        qp[h][0] = c.x;
        qp[h][1] = c.y;
        qp[h][2] = c.z;
        qp[h][3] = c.w;
      }
    }
    const float sl = a.scale_log2;
    const uint16_t *kbase = static_cast<const uint16_t *>(a.k_cache);
    const uint16_t *vbase = static_cast<const uint16_t *>(a.v_cache);
    const uint32_t lane_bytes = (uint32_t)(((size_t)kvh * D + (size_t)col * 8) * 2);
    const uint32_t vlane_bytes = (uint32_t)(((size_t)kvh * DV + (size_t)col * EV) * 2);
    const ro_i32_ptr tab = read_only(a.block_tables + (size_t)seq * a.max_blocks_per_seq);

    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EV; ++e) acc[h][e] = 0.f;

    const int ntok = p1 - p0;
    const int nchunks = ntok > 0 ? (ntok + U - 1) / U : 0;
    // Software pipeline: a wave's next step (c + W) has its K and V loads
    // in flight while the current step is computed, two register sets
    // taking turns.
    Step sa, sb;
    int c = wave;
    if (c >= nchunks) return;
    issue(a, tab, p0, p1, c, kbase, vbase, lane_bytes, vlane_bytes, sa);
    while (true) {
      if (c + W < nchunks) issue(a, tab, p0, p1, c + W, kbase, vbase, lane_bytes, vlane_bytes, sb);
      consume(sa, qp, sl, col, m, l, acc);
      c += W;
      if (c >= nchunks) break;
      if (c + W < nchunks) issue(a, tab, p0, p1, c + W, kbase, vbase, lane_bytes, vlane_bytes, sa);
      consume(sb, qp, sl, col, m, l, acc);
      c += W;
      if (c >= nchunks) break;
    }
  }

  // One wave step's loaded rows: U tokens' K (16 bytes per lane) and V
  // slices, and whether each token is inside the range and its block id
  // inside the pool.
  struct Step {
    uint4 kr[U];
    uint32_t vr[U][VW];
    bool ok[U];
  };

  // Issue the loads of step c (tokens p0 + c*U ..): token u's slot (0,
  // the pool start, when it lies past the range or in a block outside the
  // pool), the same for the whole wave.
  __device__ static __forceinline__ void issue(const DecodeKernelArgs &a, ro_i32_ptr tab, int p0, int p1, int c,
                                               const uint16_t *kbase, const uint16_t *vbase, uint32_t lane_bytes,
                                               uint32_t vlane_bytes, Step &st) {
    const int shift = a.block_shift;
    const int bs_mask = (1 << shift) - 1;
    const size_t slot_stride = (size_t)a.num_kv_heads * D;    // K elements per token slot
    const size_t vslot_stride = (size_t)a.num_kv_heads * DV;  // V elements per token slot
    const int cbase = p0 + c * U;
    size_t off[U], voff[U];
    int blk[U];
#pragma unroll
    for (int u = 0; u < U; ++u) blk[u] = tab[min((cbase + u) >> shift, a.max_blocks_per_seq - 1)];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int tok = cbase + u;
      st.ok[u] = (tok < p1) && ((unsigned)blk[u] < (unsigned)a.num_blocks);
      const size_t slot = st.ok[u] ? (((size_t)(uint32_t)blk[u] << shift) + (size_t)(tok & bs_mask)) : 0;
      off[u] = slot * slot_stride;
      voff[u] = slot * vslot_stride;
    }
    chunk_load<U>(st.kr, off, kbase, lane_bytes);
    chunk_load_words<U, VW>(st.vr, voff, vbase, vlane_bytes);
  }

  // Scores, online softmax and P.V of one loaded step.
  __device__ static __forceinline__ void consume(Step &st, const uint32_t (&qp)[G][4], float sl, int col, float &m,
                                                 float &l, float (&acc)[G][EV]) {
    float s[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float d[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float t = dot2_bf16(qp[h][0], st.kr[u].x, 0.f);
        t = dot2_bf16(qp[h][1], st.kr[u].y, t);
        t = dot2_bf16(qp[h][2], st.kr[u].z, t);
        d[h] = dot2_bf16(qp[h][3], st.kr[u].w, t);
      }
      const float r = row_scatter_sum<L, G>(d);
      s[u] = st.ok[u] ? r * sl : -INFINITY;
    }
    float cm = s[0];
#pragma unroll
    for (int u = 1; u < U; ++u) cm = fmaxf(cm, s[u]);
    // lazy rescale, per lane (each lane's row is one kv head; the lanes
    // of a row with the same head index hold the same values)
    const bool grow = cm > m + kDecodeRescaleSlack;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float alpha = grow ? fast_exp2(m - cm) : 1.f;  // 0 when m is -inf
      m = grow ? cm : m;
      l *= alpha;
      float ah[G];
      every_head<G>(alpha, col, ah);
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EV; ++e) acc[h][e] *= ah[h];
    }
    float p[U];
    float psum = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      p[u] = st.ok[u] ? fast_exp2(s[u] - m) : 0.f;
      psum += p[u];
    }
    l += psum;
    // a token outside the range (or in an invalid block) may hold
    // anything, NaN included: zero its V so that weight 0 gives exactly 0
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (!st.ok[u]) {
#pragma unroll
        for (int j = 0; j < VW; ++j) st.vr[u][j] = 0;
      }
#pragma unroll
    for (int u = 0; u < U; u += 2) {
      uint32_t vp[EV];
#pragma unroll
      for (int j = 0; j < VW; ++j) {
        vp[2 * j] = interleave_lo(st.vr[u][j], st.vr[u + 1][j]);
        vp[2 * j + 1] = interleave_hi(st.vr[u][j], st.vr[u + 1][j]);
      }
      uint32_t pk[G];
      every_head<G>(pack_bf16x2_rne(p[u], p[u + 1]), col, pk);
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < EV; ++e) acc[h][e] = dot2_bf16(pk[h], vp[e], acc[h][e]);
    }
  }

  // The newest token of sequence `seq` (position pos) from the fused-append
  // input rows, added to wave 0's totals for every kv head of its rows, and
  // its rows written into the token's cache slot (see Bf16Decode).
  __device__ static __forceinline__ void attend_new(const DecodeKernelArgs &a, int seq, int kvh0, int pos,
                                                    int lane, float &m, float &l, float (&acc)[G][EV]) {
    const int col = lane % L;
    const int kvh = lane_head(a, kvh0, lane);
    const bool row_ok = kvh0 + lane / L < a.num_kv_heads;
    const int blk = read_only(a.block_tables + (size_t)seq * a.max_blocks_per_seq)[pos >> a.block_shift];
    if ((unsigned)blk >= (unsigned)a.num_blocks) return;
    const size_t in_row = ((size_t)seq * a.num_kv_heads + kvh) * D + (size_t)col * 8;
    const size_t in_vrow = ((size_t)seq * a.num_kv_heads + kvh) * DV + (size_t)col * EV;
    const uint4 kc = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.new_k) + in_row);
    Vec<bf16_t, EV> vc;
    vc.load(static_cast<const bf16_t *>(a.new_v) + in_vrow);
    const uint4 *qv = reinterpret_cast<const uint4 *>(
        static_cast<const uint16_t *>(a.q) + ((size_t)seq * a.num_heads + (size_t)kvh * G) * D);
    float d[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const uint4 qc = qv[(h ^ (col & (G - 1))) * L + col];  // slot h: head h ^ (col % G)
      float t = dot2_bf16(qc.x, kc.x, 0.f);
      t = dot2_bf16(qc.y, kc.y, t);
      t = dot2_bf16(qc.z, kc.z, t);
      d[h] = dot2_bf16(qc.w, kc.w, t);
    }
    const float s = row_scatter_sum<L, G>(d) * a.scale_log2;  // head col % G of this row's kv head
    const float m_new = fmaxf(m, s);
    const float alpha = fast_exp2(m - m_new);  // 0 while m is still -inf
    const float p = fast_exp2(s - m_new);
    m = m_new;
    l = l * alpha + p;
    float vf[EV];
    vc.widen(vf);
    float ah[G], pb[G];
    every_head<G>(alpha, col, ah);
    every_head<G>(p, col, pb);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float pr = bf16_lo(pack_bf16x2_rne(pb[h], 0.f));  // the weight rounded to bf16
#pragma unroll
      for (int e = 0; e < EV; ++e) acc[h][e] = fmaf(pr, vf[e], acc[h][e] * ah[h]);
    }
    if (row_ok) {
      const size_t slot = ((size_t)blk << a.block_shift) + (size_t)(pos & ((1 << a.block_shift) - 1));
      const size_t at = slot * a.num_kv_heads * D + (size_t)kvh * D + (size_t)col * 8;
      const size_t vat = slot * a.num_kv_heads * DV + (size_t)kvh * DV + (size_t)col * EV;
      *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(const_cast<void *>(a.k_cache)) + at) = kc;
      uint32_t *vdst = reinterpret_cast<uint32_t *>(static_cast<uint16_t *>(const_cast<void *>(a.v_cache)) + vat);
      if constexpr (VW == 2) {
        *reinterpret_cast<uint2 *>(vdst) = make_uint2(vc.w[0], vc.w[1]);
      } else {
#pragma unroll
        for (int i = 0; i < VW / 4; ++i)
          reinterpret_cast<uint4 *>(vdst)[i] = make_uint4(vc.w[4 * i], vc.w[4 * i + 1], vc.w[4 * i + 2], vc.w[4 * i + 3]);
      }
    }
  }

  // The W = 4 waves' (m, l, acc) are merged in a tree through two wave
  // slots of LDS: waves 2 and 3 park theirs, waves 0 and 1 fold them in,
  // wave 1 parks the result, wave 0 folds it in and writes.  Two slots
  // instead of four keep the staging of eight heads per kv head small
  // enough for three work-groups per CU.
  static_assert(W == 4, "the merge tree takes four waves");
  struct Stage {
    float m[2][R][G];
    float l[2][R][G];
    float o[2][R][G][DV];
  };

  __device__ static __forceinline__ void put(Stage &sm, int slot, int lane, float m, float l,
                                             const float (&acc)[G][EV]) {
    const int row = lane / L;
    const int col = lane % L;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < EV; ++e) sm.o[slot][row][h][col * EV + e] = acc[h][e];
    if (col < G) {  // lane c of each row owns head c
      sm.m[slot][row][col] = m;
      sm.l[slot][row][col] = l;
    }
  }

  // this wave's totals merged with a parked slot's: M = max(m, m'),
  // o = o 2^(m - M) + o' 2^(m' - M), l likewise (a side with no token has
  // m = -inf and weight 0)
  __device__ static __forceinline__ void merge(const Stage &sm, int slot, int lane, float &m, float &l,
                                               float (&acc)[G][EV]) {
    const int row = lane / L;
    const int col = lane % L;
    float mh[G];
    every_head<G>(m, col, mh);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float ms = sm.m[slot][row][h];
      const float M = fmaxf(mh[h], ms);
      const float fa = mh[h] == -INFINITY ? 0.f : fast_exp2(mh[h] - M);
      const float fb = ms == -INFINITY ? 0.f : fast_exp2(ms - M);
#pragma unroll
      for (int e = 0; e < EV; ++e) acc[h][e] = fmaf(sm.o[slot][row][h][col * EV + e], fb, acc[h][e] * fa);
    }
    const int hh = col % G;  // this lane's own head
    const float ms = sm.m[slot][row][hh];
    const float M = fmaxf(m, ms);
    const float fa = m == -INFINITY ? 0.f : fast_exp2(m - M);
    const float fb = ms == -INFINITY ? 0.f : fast_exp2(ms - M);
    l = fmaf(sm.l[slot][row][hh], fb, l * fa);
    m = M;
  }

  // The merged totals of one wave: the output rows o / l (`direct`) or the
  // partial (o, m, l) of partition slot `slot`, for every row's kv head
  // below num_kv_heads.  Lane (row, col) holds dims col*EV .. col*EV+EV-1
  // of every head of its row.
  __device__ static __forceinline__ void write(const DecodeKernelArgs &a, int seq, int kvh0, int lane, float m,
                                               float l, const float (&acc)[G][EV], bool direct, int slot) {
    const int row = lane / L;
    const int col = lane % L;
    float lh[G];
    every_head<G>(l, col, lh);
    const int kvh = kvh0 + row;
    if (kvh >= a.num_kv_heads) return;  // rows past the last kv head
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const size_t head = (size_t)seq * a.num_heads + (size_t)kvh * G + h;
      if (direct) {
        uint32_t w[EV / 2];
#pragma unroll
        for (int j = 0; j < EV / 2; ++j) {
          const float r0 = lh[h] > 0.f ? acc[h][2 * j] / lh[h] : 0.f;
          const float r1 = lh[h] > 0.f ? acc[h][2 * j + 1] / lh[h] : 0.f;
          w[j] = pack_bf16x2(r0, r1);
        }
        uint16_t *dst = static_cast<uint16_t *>(a.out) + head * DV + (size_t)col * EV;
        if constexpr (EV == 8) {
          *reinterpret_cast<uint4 *>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
        } else {
#pragma unroll
          for (int j = 0; j < EV / 4; ++j) reinterpret_cast<uint2 *>(dst)[j] = make_uint2(w[2 * j], w[2 * j + 1]);
        }
      } else {
        const size_t idx = head * a.max_partitions + slot;
        float4 *dst = reinterpret_cast<float4 *>(a.ws_o + idx * DV + (size_t)col * EV);
#pragma unroll
        for (int j = 0; j < EV / 4; ++j)
          dst[j] = make_float4(acc[h][4 * j], acc[h][4 * j + 1], acc[h][4 * j + 2], acc[h][4 * j + 3]);
        if (col == h) {  // the lane whose own head is h
          a.ws_m[idx] = m;
          a.ws_l[idx] = l;
        }
      }
    }
  }
};

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
  const int ctx = lane < S ? decode_context(a, lane) : 0;
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

template <int D, int DV, int G>
__global__ void __launch_bounds__(64 * kDecodeWaves)
// four work-groups per CU while the accumulators fit (up to G = 4 at DV <= D)
__attribute__((amdgpu_waves_per_eu((G <= 4 && G * (DV / (D / 8)) <= 32) ? 4 : 1)))
decode_partition_bf16_kernel(const DecodeKernelArgs a) {
  using K = Bf16Decode<D, DV, G>;
  constexpr int W = K::W;
  const int kvh = blockIdx.x;
  int seq = blockIdx.y;
  int part = blockIdx.z;
  if (a.group_start == nullptr && a.partition_size > 0 && a.num_seqs <= 64) {
    __shared__ int s_map[2];
    if (threadIdx.x < 64) {
      int sq = 0, pt = 0;
      const bool ok = size_order_item(a, blockIdx.z * gridDim.y + blockIdx.y, threadIdx.x, sq, pt);
      if (threadIdx.x == 0) {
        s_map[0] = ok ? sq : 0;
        s_map[1] = ok ? pt : a.max_partitions;  // no pair: past every sequence's partitions
      }
    }
    __syncthreads();
    // uniform over the work-group: kept in scalar registers, so that every
    // address derived from them is a scalar base plus the lane's offset
    seq = __builtin_amdgcn_readfirstlane(s_map[0]);
    part = __builtin_amdgcn_readfirstlane(s_map[1]);
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave

  const int ctx = decode_context(a, seq);
  // cascade: this launch covers the row's own tokens after the shared ones,
  // into the partition slots after those of the shared chunks
  const bool cascade = a.group_start != nullptr;
  const int sh = decode_shared(a, seq, ctx);
  const int nparts = cascade ? (ctx - sh + a.partition_size - 1) / a.partition_size
                             : decode_num_partitions(a, ctx);
  if (part >= nparts) return;
  const int ps = a.partition_size > 0 ? a.partition_size : ctx;
  const int p0 = sh + part * ps;
  const int p1 = min(ctx, p0 + ps);
  const int slot = cascade ? (sh + a.shared_chunk - 1) / a.shared_chunk + part : part;

  // fused append: the newest token comes from the input rows, in wave 0,
  // after the cached tokens
  const bool append = a.new_k != nullptr && !cascade && part == nparts - 1 && ctx > 0;
  float m, l, acc[G][K::EV];
  K::attend(a, seq, kvh, p0, append ? p1 - 1 : p1, wave, lane, m, l, acc);
  if (append && wave == 0) K::attend_new(a, seq, kvh, ctx - 1, lane, m, l, acc);

  __shared__ typename K::Stage sm;
  K::stage(sm, wave, lane, m, l, acc);
  __syncthreads();

  const bool direct = !cascade && nparts == 1;
  for (int i = threadIdx.x; i < G * DV; i += 64 * W) {
    float M, o, lt;
    K::combine(sm, i, M, o, lt);
    const int head = kvh * G + i / DV;
    const int d = i % DV;
    if (direct) {
      const float r = (lt > 0.f) ? o / lt : 0.f;
      store_one<bf16_t>(a.out, ((size_t)seq * a.num_heads + head) * DV + d, r);
    } else {
      const size_t idx = ((size_t)seq * a.num_heads + head) * a.max_partitions + slot;
      a.ws_o[idx * DV + d] = o;
      if (d == 0) {
        a.ws_m[idx] = M;
        a.ws_l[idx] = lt;
      }
    }
  }
}

// The partition kernel on Bf16DecodeRows: work-group (kv head group,
// sequence, partition), the kv head group being R consecutive kv heads.
template <int D, int DV, int G>
__global__ void __launch_bounds__(64 * kDecodeWaves)
// three work-groups per CU while the two steps' rows and the accumulators
// fit (up to G = 4 at DV <= D)
__attribute__((amdgpu_waves_per_eu((G <= 4 && G * (DV / (D / 8)) <= 32) ? 3 : 1)))
decode_partition_rows_kernel(const DecodeKernelArgs a) {
  using K = Bf16DecodeRows<D, DV, G>;
  constexpr int R = K::R;
  const int kvh0 = blockIdx.x * R;
  int seq = blockIdx.y;
  int part = blockIdx.z;
  if (a.group_start == nullptr && a.partition_size > 0 && a.num_seqs <= 64) {
    __shared__ int s_map[2];
    if (threadIdx.x < 64) {
      int sq = 0, pt = 0;
      const bool ok = size_order_item(a, blockIdx.z * gridDim.y + blockIdx.y, threadIdx.x, sq, pt);
      if (threadIdx.x == 0) {
        s_map[0] = ok ? sq : 0;
        s_map[1] = ok ? pt : a.max_partitions;  // no pair: past every sequence's partitions
      }
    }
    __syncthreads();
    // uniform over the work-group: kept in scalar registers, so that every
    // address derived from them is a scalar base plus the lane's offset
    seq = __builtin_amdgcn_readfirstlane(s_map[0]);
    part = __builtin_amdgcn_readfirstlane(s_map[1]);
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave

  const int ctx = decode_context(a, seq);
  const bool cascade = a.group_start != nullptr;
  const int sh = decode_shared(a, seq, ctx);
  const int nparts = cascade ? (ctx - sh + a.partition_size - 1) / a.partition_size
                             : decode_num_partitions(a, ctx);
  if (part >= nparts) return;
  const int ps = a.partition_size > 0 ? a.partition_size : ctx;
  const int p0 = sh + part * ps;
  const int p1 = min(ctx, p0 + ps);
  const int slot = cascade ? (sh + a.shared_chunk - 1) / a.shared_chunk + part : part;

  const bool append = a.new_k != nullptr && !cascade && part == nparts - 1 && ctx > 0;
  float m, l, acc[G][K::EV];
  K::attend(a, seq, kvh0, p0, append ? p1 - 1 : p1, wave, lane, m, l, acc);
  if (append && wave == 0) K::attend_new(a, seq, kvh0, ctx - 1, lane, m, l, acc);

  __shared__ typename K::Stage sm;
  if (wave >= 2) K::put(sm, wave - 2, lane, m, l, acc);
  __syncthreads();
  if (wave < 2) K::merge(sm, wave, lane, m, l, acc);
  __syncthreads();
  if (wave == 1) K::put(sm, 0, lane, m, l, acc);
  __syncthreads();
  if (wave == 0) {
    K::merge(sm, 0, lane, m, l, acc);
    K::write(a, seq, kvh0, lane, m, l, acc, !cascade && nparts == 1, slot);
  }
}

// ------------------------------------------------------------------------
// Matrix-core decode (bf16, key and value head dim 128).  Per kv head, the
// scores of a tile of 16 tokens and the tile's share of the weighted sum
// are two small matrix products:
//   S^T = K Q^T    on v_mfma_f32_16x16x32_bf16 (16 tokens x 16 columns, the
//                  G query heads of the kv head as columns, the rest zero),
//   O^T += V^T P^T on v_mfma_f32_16x16x16_bf16 (value dims x columns).
// In the accumulator layout lane l holds column l % 16 and tokens
// 4 (l / 16) .. 4 (l / 16) + 3 of S^T, which is also the B operand layout
// of the second product, so the weights go from the exponentials straight
// into the products.  The vector work per token (a scale, an exponential,
// the max and the sum, shared by up to 16 heads) no longer grows with G.
//  * One wave per kv head: a work-group (4 waves) covers 4 consecutive kv
//    heads of one (sequence, partition), every wave all of the partition's
//    tokens; no cross-wave merge.
//  * A tile is loaded row-major, 4 tokens x the kv head's 256-byte row per
//    load instruction (a scalar block id per instruction: a load's 4 tokens
//    start at a multiple of 4 and share one block), into registers, and
//    from there into the wave's own LDS slice; the registers then take the
//    next tile's loads, which are in flight while the staged tile is
//    computed.  One register set per wave leaves room for four work-groups
//    per CU.  The score product reads K from LDS with one 16-byte read per
//    lane and k-step, the value product V^T with gfx950's transposing 8-byte
//    reads.  Rows are padded (K 272 bytes, V 288 bytes) so that both kinds
//    of reads hit distinct banks.
//  * Tokens outside the range, or in a block outside the pool, are
//    selected out: score -inf, weight 0, and their V rows zeroed before
//    they enter the product, whatever the slot holds.
//  * The running max is a reference moved only when a tile exceeds it by
//    more than 2^8, as in the row-layout kernel; the running sum takes the
//    fp32 weights, the products their bf16 roundings (nearest even).
//  * Fused append: the newest token's rows come from the input rows (they
//    replace the loaded slot contents in registers) and are written into
//    its slot after the last tile.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) u32x4_t *lds_u4_ptr;
typedef __attribute__((address_space(3))) const bf16x8_t *lds_b8_ptr;
typedef __attribute__((address_space(3))) v4i16_t *lds_v4_ptr;

template <int G, int TT = 16>
struct Bf16DecodeMfma {
  static constexpr int D = 128;
  static constexpr int DV = 128;
  static constexpr int MT = TT / 16;   // 16-token sub-tiles per tile
  static constexpr int NL = TT / 4;    // K (and V) load instructions per tile: 4 tokens x 256 B each
  static constexpr int NKS = D / 32;   // k-steps of the score product
  static constexpr int NDT = DV / 16;  // 16-row tiles of O^T
  static constexpr int KROW = 272;     // LDS bytes per K row: 16 rows at one chunk cover every bank
  static constexpr int VROW = 288;     // LDS bytes per V row: the transposing reads of 8 rows cover every bank
  static constexpr int KBYTES = TT * KROW;
  static constexpr int LDS_BYTES = KBYTES + TT * VROW;  // one wave's slice
  static_assert(TT % 16 == 0, "tiles of whole 16-token sub-tiles");
  static_assert(G >= 1 && G <= 16, "the query heads of a kv head are columns of a 16-wide tile");

  // One tile's rows: load j holds tokens t0 + 4j .. t0 + 4j + 3 (lane l:
  // token t0 + 4j + l / 16, 16-byte chunk l % 16 of its row); bit j of ok:
  // load j's first token is in range and its block inside the pool.
  struct Tile {
    uint4 k[NL];
    uint4 v[NL];
    int ok;
  };

  __device__ static __forceinline__ void issue(const DecodeKernelArgs &a, ro_i32_ptr tab, int t0, int p1,
                                               const char *kbase, const char *vbase, uint32_t lane_off,
                                               size_t slot_bytes, Tile &t) {
    const int shift = a.block_shift;
    const int bs_mask = (1 << shift) - 1;
    int blk[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) blk[j] = tab[min((t0 + 4 * j) >> shift, a.max_blocks_per_seq - 1)];
    int ok = 0;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      const int tok = t0 + 4 * j;
      const bool good = (tok < p1) && ((unsigned)blk[j] < (unsigned)a.num_blocks);
      ok |= good ? (1 << j) : 0;
      // a load that is not attended reads the pool's first slots
      const size_t off = good ? (((size_t)(uint32_t)blk[j] << shift) + (size_t)(tok & bs_mask)) * slot_bytes : 0;
      const u32x4_t kv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(kbase + off + lane_off));
      const u32x4_t vv = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(vbase + off + lane_off));
      t.k[j] = make_uint4(kv.x, kv.y, kv.z, kv.w);
      t.v[j] = make_uint4(vv.x, vv.y, vv.z, vv.w);
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
  // padded rows).  Rows that are not attended get a zero V row; the
  // appended token's rows come from the input.
  __device__ static __forceinline__ void stage(Tile &t, int t0, int p1, int pnew, uint4 kn, uint4 vn, int lane,
                                               uint32_t lds) {
    const int g = lane >> 4;
    const int c = lane & 15;
    if (t.ok != (1 << NL) - 1 || t0 + TT > p1) {
#pragma unroll
      for (int j = 0; j < NL; ++j)
        if (!(((t.ok >> j) & 1) && t0 + 4 * j + g < p1)) t.v[j] = make_uint4(0u, 0u, 0u, 0u);
    }
    if (pnew >= t0 && pnew < t0 + TT) {
      const int tl = pnew - t0;
#pragma unroll
      for (int j = 0; j < NL; ++j)
        if (j == (tl >> 2) && g == (tl & 3) && ((t.ok >> j) & 1)) {
          t.k[j] = kn;
          t.v[j] = vn;
        }
    }
    const uint32_t kw = lds + (uint32_t)(g * KROW + c * 16);
    const uint32_t vw = lds + (uint32_t)(KBYTES + g * VROW + c * 16);
#pragma unroll
    for (int j = 0; j < NL; ++j) {
      *(lds_u4_ptr)(size_t)(kw + j * 4 * KROW) = u32x4_t{t.k[j].x, t.k[j].y, t.k[j].z, t.k[j].w};
      *(lds_u4_ptr)(size_t)(vw + j * 4 * VROW) = u32x4_t{t.v[j].x, t.v[j].y, t.v[j].z, t.v[j].w};
    }
  }

  // Scores, online softmax and P.V of the tile at tokens t0 .. staged in
  // LDS (ok: its loads' bits).
  __device__ static __forceinline__ void compute(int ok, int t0, int p1, float sl, int lane, uint32_t lds,
                                                 State &st) {
    const int g = lane >> 4;
    const int c = lane & 15;
    // S^T = K Q^T per sub-tile: A = K rows (lane: token 16 mt + c, chunk
    // 4 ks + g)
    const uint32_t kr = lds + (uint32_t)(c * KROW + g * 16);
    f32x4_t s[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      s[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const bf16x8_t kf = *(lds_b8_ptr)(size_t)(kr + mt * 16 * KROW + ks * 64);
        s[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, st.qf[ks], s[mt], 0, 0, 0);
      }
    }
    // weights of column c for tokens 16 mt + 4g .. 16 mt + 4g + 3 (loaded
    // by load 4 mt + g)
    float sv[MT][4];
    bool vok[MT][4];
    float cm = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const bool row_ok = (ok >> (4 * mt + g)) & 1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        vok[mt][r] = row_ok && (t0 + 16 * mt + 4 * g + r < p1);
        sv[mt][r] = vok[mt][r] ? s[mt][r] * sl : -INFINITY;
        cm = fmaxf(cm, sv[mt][r]);
      }
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
    // O^T += V^T P^T per sub-tile: A = V^T from transposing reads.  In
    // 16-lane group g, lane c sends the address of 4 value dims of one
    // token (token 16 mt + 4g + c / 4, dims 16 dt + 4 (c % 4)) and receives
    // dim 16 dt + c of tokens 16 mt + 4g .. 16 mt + 4g + 3.
    const uint32_t vr = lds + (uint32_t)(KBYTES + (4 * g + (c >> 2)) * VROW + (c & 3) * 8);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = vok[mt][r] ? fast_exp2(sv[mt][r] - st.m) : 0.f;
      st.l += (p[0] + p[1]) + (p[2] + p[3]);
      const uint32_t p01 = pack_bf16x2_rne(p[0], p[1]);
      const uint32_t p23 = pack_bf16x2_rne(p[2], p[3]);
      const v4i16_t pb = __builtin_bit_cast(v4i16_t, make_uint2(p01, p23));
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const v4i16_t vf =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4_ptr)(size_t)(vr + mt * 16 * VROW + dt * 32));
        st.o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf, pb, st.o[dt], 0, 0, 0);
      }
    }
  }

  // Online softmax of kv head kvh's query heads over tokens p0 .. p1-1 of
  // sequence seq; pnew (or -1): the appended token, whose rows are kn, vn.
  __device__ static __forceinline__ void attend(const DecodeKernelArgs &a, int seq, int kvh, int p0, int p1,
                                                int pnew, uint4 kn, uint4 vn, int lane, uint32_t lds, State &st) {
    const int g = lane >> 4;
    const int c = lane & 15;
    {
      const uint4 *qrow = reinterpret_cast<const uint4 *>(
          static_cast<const uint16_t *>(a.q) + ((size_t)seq * a.num_heads + (size_t)kvh * G + (c < G ? c : 0)) * D);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const uint4 w = c < G ? qrow[4 * ks + g] : make_uint4(0u, 0u, 0u, 0u);
        st.qf[ks] = __builtin_bit_cast(bf16x8_t, w);
      }
    }
    st.m = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) st.o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int ntiles = p1 > p0 ? (p1 - p0 + TT - 1) / TT : 0;
    if (ntiles == 0) return;

    const float sl = a.scale_log2;
    const size_t slot_bytes = (size_t)a.num_kv_heads * D * 2;
    const uint32_t lane_off = (uint32_t)((size_t)g * slot_bytes + (size_t)kvh * D * 2 + (size_t)c * 16);
    const char *kbase = static_cast<const char *>(a.k_cache);
    const char *vbase = static_cast<const char *>(a.v_cache);
    const ro_i32_ptr tab = read_only(a.block_tables + (size_t)seq * a.max_blocks_per_seq);
    // One register set: once a tile is in LDS its registers take the next
    // tile's loads, which are in flight while the staged tile is computed.
    Tile t;
    issue(a, tab, p0, p1, kbase, vbase, lane_off, slot_bytes, t);
    for (int i = 0; i < ntiles; ++i) {
      const int t0 = p0 + i * TT;
      stage(t, t0, p1, pnew, kn, vn, lane, lds);
      const int ok = t.ok;
      if (i + 1 < ntiles) issue(a, tab, t0 + TT, p1, kbase, vbase, lane_off, slot_bytes, t);
      compute(ok, t0, p1, sl, lane, lds, st);
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

// The partition kernel on Bf16DecodeMfma: work-group (group of 4 kv heads,
// sequence, partition) in the size order of the row-layout kernel, one
// wave per kv head.  Plain decode only (no cascade).
template <int G>
__global__ void __launch_bounds__(64 * kDecodeWaves)
// four work-groups per CU (one tile's rows in registers per wave, 35 KB of
// LDS per work-group)
__attribute__((amdgpu_waves_per_eu(4)))
decode_partition_mfma_kernel(const DecodeKernelArgs a) {
  using K = Bf16DecodeMfma<G>;
  int seq = blockIdx.y;
  int part = blockIdx.z;
  if (a.partition_size > 0 && a.num_seqs <= 64) {
    __shared__ int s_map[2];
    if (threadIdx.x < 64) {
      int sq = 0, pt = 0;
      const bool ok = size_order_item(a, blockIdx.z * gridDim.y + blockIdx.y, threadIdx.x, sq, pt);
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

  const int ctx = decode_context(a, seq);
  const int nparts = decode_num_partitions(a, ctx);
  if (part >= nparts) return;
  const int ps = a.partition_size > 0 ? a.partition_size : ctx;
  const int p0 = part * ps;
  const int p1 = min(ctx, p0 + ps);

  // fused append: the newest token's rows from the input rows
  const bool append = a.new_k != nullptr && part == nparts - 1 && ctx > 0;
  const int pnew = append ? ctx - 1 : -1;
  uint4 kn = make_uint4(0u, 0u, 0u, 0u), vn = kn;
  if (append) {
    const size_t in_row = ((size_t)seq * a.num_kv_heads + kvh) * K::D + (size_t)(lane & 15) * 8;
    kn = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.new_k) + in_row);
    vn = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.new_v) + in_row);
  }

  __shared__ __attribute__((aligned(16))) char lds[kDecodeWaves][K::LDS_BYTES];
  typedef __attribute__((address_space(3))) char *lds_char_ptr;
  const uint32_t my_lds = (uint32_t)(size_t)(lds_char_ptr)(&lds[wave][0]);
  typename K::State st;
  K::attend(a, seq, kvh, p0, p1, pnew, kn, vn, lane, my_lds, st);

  if (append && lane < 16) {
    // the appended rows into the token's slot (after every load of this
    // wave has been consumed); a block outside the pool is skipped
    const int blk = read_only(a.block_tables + (size_t)seq * a.max_blocks_per_seq)[pnew >> a.block_shift];
    if ((unsigned)blk < (unsigned)a.num_blocks) {
      const size_t slot = ((size_t)blk << a.block_shift) + (size_t)(pnew & ((1 << a.block_shift) - 1));
      const size_t at = (slot * a.num_kv_heads + kvh) * K::D + (size_t)lane * 8;
      *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(const_cast<void *>(a.k_cache)) + at) = kn;
      *reinterpret_cast<uint4 *>(static_cast<uint16_t *>(const_cast<void *>(a.v_cache)) + at) = vn;
    }
  }
  K::write(a, seq, kvh, lane, st, nparts == 1, part);
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
  k.query_start_loc = a.query_start_loc;
  k.num_prefill_seqs = a.num_prefill_seqs;
  k.new_k = a.new_k;
  k.new_v = a.new_v;
  return k;
}

template <typename T, int D, int DV, int G>
static hipError_t launch_partition_t(const DecodeArgs &a, hipStream_t stream) {
  const DecodeKernelArgs k = make_kernel_args(a);
  dim3 grid(a.max_partitions, a.cache.num_kv_heads, a.num_seqs);
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (a.query_start_loc) return hipErrorNotSupported;  // prefill rows run on the generic kernel only
    if constexpr (D == 128 && DV == 128) {
      // plain decode at head dims 128 on the matrix cores; the own-token
      // pass of cascade decode below, on the row-layout kernel
      if (!a.group_start) {
        grid = dim3((a.cache.num_kv_heads + kDecodeWaves - 1) / kDecodeWaves, a.num_seqs, a.max_partitions);
        hipLaunchKernelGGL((decode_partition_mfma_kernel<G>), grid, dim3(64 * kDecodeWaves), 0, stream, k);
        return hipGetLastError();
      }
    }
    if constexpr (D == 128) {
      // rows across kv heads: R = 4 kv heads per work-group
      constexpr int R = Bf16DecodeRows<D, DV, G>::R;
      grid = dim3((a.cache.num_kv_heads + R - 1) / R, a.num_seqs, a.max_partitions);
      hipLaunchKernelGGL((decode_partition_rows_kernel<D, DV, G>), grid, dim3(64 * kDecodeWaves), 0, stream, k);
    } else {
      grid = dim3(a.cache.num_kv_heads, a.num_seqs, a.max_partitions);
      hipLaunchKernelGGL((decode_partition_bf16_kernel<D, DV, G>), grid, dim3(64 * kDecodeWaves), 0, stream, k);
    }
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
