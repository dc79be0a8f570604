// Paged-attention decode kernel for gfx950 (MI355X).
//
// Work decomposition. Every (sequence s, kv head g, tile of <= 16 query heads) is one *stream* of
// nb_s = ceil(n_s / 16) blocks. The streams are laid end to end, (kv head, head tile)-major and
// then by sequence, into one flattened space of W = sum_s nb_s * (kv heads * head tiles) block
// positions, and the launch's workgroups cut that space into contiguous ranges: equal ones, or
// (when the equal cut would split streams anyway) ranges weighted by the XCD a workgroup runs on,
// since odd-numbered XCDs stream measurably slower (see range_start). Consecutive ranges run on
// one XCD (range_of_workgroup), so the sequences of one kv head -- and the blocks they share, such
// as a common prompt prefix -- are read through one L2. When the library chose the full grid and
// the batch has no more streams than workgroups, of uneven lengths, only the first half of the
// workgroups (one per compute unit) take ranges, which halves the streams the cut splits. A
// workgroup's share is thus fixed whatever the mix of context lengths: a 32k-token sequence is
// spread over many workgroups and a batch of short ones is packed into few, with no per-sequence
// partition size to tune and no tail of idle compute units. Each workgroup derives the plan
// itself from context_lens (a prefix sum in LDS), so the host needs no device data.
//
// Inside a range the four wavefronts interleave block by block (wave i takes positions
// r0 + i, r0 + i + 4, ...), so all four always work on the same stream. Per 16-token block a
// wavefront looks up the block's physical id in the sequence's block table, row s, entry j / R
// for unit j of the stream (R = 16-token units per block; "PagedAttention and KV Cache
// Management" (blog.sejan.dev), section "Under the Hood: The PagedAttention CUDA Kernel"), and:
//   * reads the K tile and the V tile straight from the pool: 64 lanes x 16 bytes per load
//     instruction, each instruction one contiguous 1 KiB range; the pool's tile order makes
//     every lane's 16 bytes a ready matrix-core operand, so nothing is staged or shuffled;
//   * scores S[token][head] = K_tile[16 x D] . Q^T[D x 16] with D/32 v_mfma_f32_16x16x32
//     (bf16 or f16) -- all query heads of a GQA group share the one K read;
//   * keeps an online softmax with a lazily moved reference maximum: the reference m only moves
//     (and the running sum and output get rescaled) when a score exceeds it by more than 2^8,
//     so probabilities stay <= 256 and the common path needs no cross-lane traffic;
//   * accumulates O[head][dim] += P[head][token] . V_tile[token][dim] with v_mfma_f32_16x16x16:
//     against bf16 V, P split into a bf16 high part and a bf16 residual, so the product keeps
//     fp32-level precision of P; against fp16 V (fp16 pools, and fp8 pools widened to fp16), one
//     fp16 P, whose 11-bit significand keeps its relative error within 2^-12.
// Tiles are prefetched RING-1 blocks ahead through a ring of registers that runs across stream
// boundaries, and nothing else is read from memory on the common path: block ids come from a
// register window of 64 per wavefront, and the q rows of the range's first streams are copied
// into LDS at the start. When a stream ends, the four wavefronts combine their (m, l, O) in LDS.
// A stream that lies wholly inside the range is normalised and stored. A stream cut by a range
// boundary leaves an fp32 partial (m, l, O) in the workspace; the last of its workgroups to finish
// (an agent-scope counter, reset by that workgroup) merges all of them in range order, so the
// result does not depend on which workgroup came last. A range's first stream, cut at its start,
// is counted as soon as it ends; the stream cut at the range's end is counted after the loop.
//
// Variants (template parameters): head dim 64 or 128; bf16 or fp16 q/out; 16-bit pools or fp8
// (E4M3) pools whose codes are widened to the q type in registers, with the pool scales folded
// into the score scale and the output normalisation; and APPEND, the fused step, in which every
// workgroup first writes the new token of each stream whose last unit it owns into the pool
// (before it reads any tile), so that the main loop is the same in every variant.
//
// Softmax identity used by both combines: with per-part reference m_p, l_p = sum exp(x - m_p)
// and O_p = sum exp(x - m_p) v, the full result is
//   sum_p 2^(m_p - M) O_p / sum_p 2^(m_p - M) l_p   for any M >= max_p m_p,
// scores being kept in log2 units (x * scale * log2 e).

#include "pkv_internal.h"

namespace pkv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// A score may exceed the reference maximum by this much (log2 units) before the reference moves.
constexpr float kLazyRescale = 8.0f;

// q rows (query heads) a workgroup stages in LDS for the first streams of its range.
constexpr int kQRows = 64;
// Parts whose loads one merge round issues together.
constexpr int kMergeRound = 4;

// Tile buffers per wavefront (blocks in flight = kRing - 1), sized to stay within 256 VGPRs so
// two workgroups fit on each compute unit. The same for fp8 tiles, which hold half the bytes:
// 5, 6 and 8 slots fit at d128 but measured slower.
template <int D>
constexpr int kRing = D == 128 ? 4 : 8;

template <bool BF16>
struct Elem;

template <>
struct Elem<true> {
  static __device__ __forceinline__ f32x4 qk(u32x4 k, u32x4 q, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k),
                                                   __builtin_bit_cast(bf16x8, q), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 pv(u32x2 p, u32x2 v, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, p),
                                                     __builtin_bit_cast(i16x4, v), c, 0, 0, 0);
  }
  // p = hi + lo (+ a residual below 2^-16 |p|), both parts 16-bit, packed in lane order.
  static __device__ __forceinline__ void split(const float p[4], u32x2& hi, u32x2& lo) {
    bf16x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[e] = (__bf16)p[e];
      l[e] = (__bf16)(p[e] - (float)h[e]);
    }
    hi = __builtin_bit_cast(u32x2, h);
    lo = __builtin_bit_cast(u32x2, l);
  }
  static __device__ __forceinline__ unsigned short store(float x) {
    return __builtin_bit_cast(unsigned short, (__bf16)x);
  }
  static __device__ __forceinline__ float widen(unsigned short b) {
    return __uint_as_float((unsigned)b << 16);
  }
  // Four E4M3 codes (bytes 0..3 of w) -> four bf16 in two dwords (exact: E4M3 is a subset).
  static __device__ __forceinline__ u32x2 from_fp8(unsigned w) {
    const bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    const bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    return u32x2{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
  }
};

template <>
struct Elem<false> {
  static __device__ __forceinline__ f32x4 qk(u32x4 k, u32x4 q, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, k),
                                                  __builtin_bit_cast(f16x8, q), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 pv(u32x2 p, u32x2 v, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, p),
                                                 __builtin_bit_cast(f16x4, v), c, 0, 0, 0);
  }
  static __device__ __forceinline__ void split(const float p[4], u32x2& hi, u32x2& lo) {
    f16x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[e] = (_Float16)p[e];
      l[e] = (_Float16)(p[e] - (float)h[e]);
    }
    hi = __builtin_bit_cast(u32x2, h);
    lo = __builtin_bit_cast(u32x2, l);
  }
  // p rounded to fp16 (11-bit significand: relative error at most 2^-12), packed in lane order.
  static __device__ __forceinline__ u32x2 round(const float p[4]) {
    f16x4 h;
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = (_Float16)p[e];
    return __builtin_bit_cast(u32x2, h);
  }
  static __device__ __forceinline__ unsigned short store(float x) {
    return __builtin_bit_cast(unsigned short, (_Float16)x);
  }
  static __device__ __forceinline__ float widen(unsigned short b) {
    return (float)__builtin_bit_cast(_Float16, b);
  }
  // Four E4M3 codes -> four fp16 (exact: every E4M3 value is an fp16 value).
  static __device__ __forceinline__ u32x2 from_fp8(unsigned w) {
    const f16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
    const f16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
    return u32x2{__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi)};
  }
};

__device__ __forceinline__ u32x4 load16(const char* p) { return *(const u32x4*)p; }

// K/V tiles are streamed: each is read once per launch, so the loads carry the non-temporal
// hint (measured on MI355X: random 4 KiB tile reads reach ~7.0 TB/s this way, ~6.2 TB/s with
// default-policy loads).
__device__ __forceinline__ u32x4 load16_stream(const char* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// s_waitcnt vmcnt(0): every vector memory access of this wave has completed. The rare loads of
// the main loop (the next stream's q, the next window of tile ids) are followed by this wait so
// that, where the paths join, only the ring's tile loads are outstanding and the compiler keeps
// the exact, deep waits of the common path.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int D, bool BF16, bool KV8, bool APPEND, int RING>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2))) void
paged_decode_kernel(DecodeLaunch a) {
  using E = Elem<BF16>;
  // Element type of the PV product. Against fp16 V -- fp16 pools, and fp8 pools, whose codes
  // widen exactly to fp16 whatever q's type -- P is one fp16 value (relative error at most
  // 2^-12). Against bf16 V it is a bf16 high part plus a bf16 residual: a bf16 P alone would
  // carry errors up to 2^-9.
  constexpr bool kSingleP = KV8 || !BF16;
  using EV = Elem<!kSingleP>;
  constexpr int NQ = D / 32;                 // QK matrix ops (32-dim chunks) per block
  constexpr int NK = KV8 ? D / 64 : D / 32;  // 16-byte K loads per block
  constexpr int NV = KV8 ? D / 64 : D / 32;  // 16-byte V loads per block
  constexpr int NO = D / 16;                 // 16-column output chunks
  constexpr size_t kTileBytes = (size_t)kBlock * D * (KV8 ? 1 : 2);  // one 16-token sub-tile
  constexpr int kRow = D + 4;  // LDS row stride (floats) of the combine buffer
  constexpr int kThreads = 64 * kWaves;
  constexpr int kHeadsPerWave = kMaxGroupTile / kWaves;   // 4 heads per wave in the combine
  constexpr int kLanesPerHead = 64 / kHeadsPerWave;       // 16
  constexpr int kDims = D / kLanesPerHead;                // 8 (d128) or 4 (d64)
  constexpr int kChunks = D / 8;                          // 16-byte chunks per q row
  constexpr int kQLoads = kQRows * kChunks / kThreads;
  // A load RING - 1 blocks ahead reads its tile id from the current or the next 64-id window.
  static_assert(RING >= 2 && RING <= 64, "prefetch must stay within the next tile-id window");

  __shared__ int s_ps[kMaxSeqs + 1];  // s_ps[s] = blocks of sequences 0..s-1
  __shared__ int s_len[kMaxSeqs];     // context lengths (clamped to the table row)
  __shared__ int s_scan[kThreads];    // scan partials; later the staged q rows' sources
  __shared__ float sm_o[kWaves][kMaxGroupTile][kRow];
  __shared__ float sm_m[kWaves][kMaxGroupTile];
  __shared__ float sm_l[kWaves][kMaxGroupTile];
  __shared__ u32x4 s_q[kQRows][kChunks];  // staged q rows of the range's first streams
  __shared__ int s_last[2];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wavefront
  const int lane = tid & 63;
  const int hl = lane & 15;    // query head within the tile (operand column)
  const int kg = lane >> 4;    // lane quarter: dims 8kg.. of each 32-dim chunk / tokens 4kg..
  const int S = a.num_seqs;

  // ---- Plan: block counts per sequence and their prefix sum, in LDS. ----
  bool same_len;  // every sequence has as many units as sequence 0
  {
    const int chunk = (S + kThreads - 1) / kThreads;
    const int lo = min(S, tid * chunk);
    const int hi = min(S, lo + chunk);
    const int nb0 = (min(max(a.context_lens[0], 0), a.max_tokens) + kBlock - 1) / kBlock;
    int sum = 0;
    bool same = true;
    for (int i = lo; i < hi; ++i) {
      const int n = min(max(a.context_lens[i], 0), a.max_tokens);
      s_len[i] = n;
      const int nb = (n + kBlock - 1) / kBlock;
      sum += nb;
      same = same && nb == nb0;
    }
    // Exclusive prefix sum of the per-thread sums: inside each wavefront by shuffles, then over
    // the wavefronts' totals (one barrier instead of two per doubling step).
    int incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    if (lane == 63) s_scan[wave] = incl;
    __syncthreads();
    int base = incl - sum;
    int total = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int t = s_scan[w];
      base += w < wave ? t : 0;
      total += t;
    }
    for (int i = lo; i < hi; ++i) {
      s_ps[i] = base;
      base += (s_len[i] + kBlock - 1) / kBlock;
    }
    if (tid == 0) s_ps[S] = total;
    same_len = __syncthreads_and(same);
  }

  // Empty sequences (n == 0) own no positions; their output is zero.
  for (int s = blockIdx.x; s < S; s += gridDim.x) {
    if (s_len[s] == 0) {
      u32x4* dst = (u32x4*)((unsigned short*)a.out + (size_t)s * a.num_q_heads * D);
      for (int c = tid; c < a.num_q_heads * D / 8; c += kThreads) dst[c] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  const int Hh = a.num_kv_heads * a.head_tiles;  // streams per sequence
  // Flattened order: (kv head, head tile) gh major, then sequence, then 16-token unit. Stream
  // (s, gh) holds positions [gh T + s_ps[s], gh T + s_ps[s + 1]), so the sequences that share
  // one kv head's blocks are neighbours in the order (and, through the XCD blocks of the ranges,
  // read on one XCD).
  const int T = uniform(s_ps[S]);  // units of one (kv head, head tile) over all sequences
  const int W = Hh * T;
  const int L = same_len ? uniform(s_ps[1] - s_ps[0]) : 0;  // units of every sequence, if equal
  // Every workgroup sees the same plan, so all decide alike.
  const RangePlan rp = plan_ranges(W, L, gridDim.x, a.may_halve, a.odd_weight);
  const int nwg = rp.nwg;
  if ((int)blockIdx.x >= nwg) return;  // uniform over the workgroup (nwg = 0: no positions)
  const int wg = range_of_workgroup(blockIdx.x, nwg);  // this workgroup's range
  const int odd_w = rp.odd_w;
  const int r0 = range_start(wg, nwg, W, odd_w);
  const int r1 = range_start(wg + 1, nwg, W, odd_w);

  // The stream holding flattened position p: gh = p / T, and the sequence s is the last one with
  // s_ps[s] <= p - gh T (empty sequences before it share its s_ps).
  auto locate = [&](int p, int& s, int& gh) {
    gh = p / T;
    const int x = p - gh * T;
    int lo = 0, hi = S;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_ps[mid] <= x) lo = mid; else hi = mid;
    }
    s = lo;
  };

  // ---- Streams (uniform cursor). ----
  struct Stream {
    int s, gh;        // sequence, kv head * head tiles + head tile
    int start, end;   // flattened positions [start, end)
    int n;            // context length
    int h0, nvalid;   // first query head of the tile, valid heads in it
  };
  auto stream_at = [&](int s, int gh) {
    Stream t;
    t.s = s;
    t.gh = gh;
    if (s < S) {
      const int pb = uniform(s_ps[s]);
      const int nb = uniform(s_ps[s + 1]) - pb;
      t.n = uniform(s_len[s]);
      t.start = gh * T + pb;
      t.end = t.start + nb;
      const int g = gh / a.head_tiles;
      const int ht = gh - g * a.head_tiles;
      t.h0 = g * a.group + ht * kMaxGroupTile;
      t.nvalid = min(kMaxGroupTile, a.group - ht * kMaxGroupTile);
    } else {  // past the last stream
      t.n = 0;
      t.start = t.end = W;
      t.h0 = 0;
      t.nvalid = 0;
    }
    return t;
  };
  auto first_nonempty = [&](int s) {
    while (s < S && uniform(s_ps[s + 1]) == uniform(s_ps[s])) ++s;  // skip empty sequences
    return s;
  };
  auto stream_after = [&](const Stream& c) {
    int s = first_nonempty(c.s + 1), gh = c.gh;
    if (s == S) {  // the next (kv head, head tile): its first non-empty sequence
      ++gh;
      s = gh < Hh ? first_nonempty(0) : S;
    }
    return stream_at(s, gh);
  };
  // The stream starting at (or holding) flattened position p.
  auto stream_from = [&](int p) {
    int s, gh;
    locate(p, s, gh);
    return stream_at(uniform(s), uniform(gh));
  };

  Stream cur = stream_from(r0);

  // ---- q: the head rows of the range's first streams, staged in LDS for all four waves. The
  // loads go out here; the rows are stored into LDS after the tile-id loads below have gone out
  // too, so that the start-up waits for one memory round trip instead of three. ----
  int staged_left;  // staged streams after the current one
  int next_qrow;    // LDS row of the next staged stream
  int q_rows;       // staged rows
  u32x4 qbuf[kQLoads];
  {
    int rows = 0, nstaged = 0;
    Stream t = cur;
    while (t.start < r1 && rows + t.nvalid <= kQRows) {
      if (tid >= rows && tid < rows + t.nvalid)
        s_scan[tid] = t.s * a.num_q_heads + t.h0 + (tid - rows);  // source row of staged row
      rows += t.nvalid;
      ++nstaged;
      t = stream_after(t);
    }
    __syncthreads();
    // Unconditional loads (rows past the staged ones reread row 0 and are not stored): no branch
    // around them, so nothing waits for them before the tile-id loads go out.
#pragma unroll
    for (int u = 0; u < kQLoads; ++u) {
      const int c = tid + kThreads * u;
      const int row = c / kChunks < rows ? c / kChunks : 0;
      qbuf[u] = load16((const char*)a.q + ((size_t)s_scan[row] * D + (c % kChunks) * 8) * 2);
    }
    staged_left = nstaged - 1;
    next_qrow = cur.nvalid;
    q_rows = rows;
  }

  // ---- Tile ids: lane l of window c holds the 16-token sub-tile of this wave's position 64c + l
  // (its index in units of 16 * D elements of the layer's K or V plane). ----
  const int span = r1 - r0;
  const int mw = span > wave ? (span - wave + kWaves - 1) / kWaves : 0;  // this wave's blocks
  // The block id of lane l's position in window c, and what the tile index adds to
  // (block id * num_kv_heads) << (sub_shift + 1): the load is issued here and used later, so
  // that several windows' loads can be in flight together.
  struct Win {
    unsigned b;    // block_tables entry (0 past the range)
    unsigned add;  // (kv head << (sub_shift + 1)) + sub-tile
  };
  auto window_load = [&](int c) -> Win {
    const int p = r0 + wave + kWaves * (64 * c + lane);
    if (p >= r1) return Win{0u, 0u};
    int s, j, g;
    if (p >= cur.start && p < cur.end) {  // in the current stream: no search, no divisions
      s = cur.s;
      j = p - cur.start;
      g = cur.gh / a.head_tiles;
    } else {
      int gh;
      locate(p, s, gh);
      j = p - gh * T - s_ps[s];
      g = gh / a.head_tiles;
    }
    // 16-token unit j of the stream: sub-tile j % R of physical block block_tables[s][j / R]
    // (R = block_size / 16 sub-tiles per block, each 16 * D elements of the block's tile). Tiles
    // of one plane lie two apart (the K and V tiles of a (block, head) alternate), so the K and V
    // sub-tile both sit at this index times 16 * D elements from their plane's base.
    return Win{(unsigned)a.block_tables[(size_t)s * a.max_blocks + (j >> a.sub_shift)],
               ((unsigned)g << (a.sub_shift + 1)) + (unsigned)(j & ((1 << a.sub_shift) - 1))};
  };
  auto tile_index = [&](const Win& w) -> unsigned {
    return ((w.b * (unsigned)a.num_kv_heads) << (a.sub_shift + 1)) + w.add;
  };
  auto window = [&](int c) -> unsigned { return tile_index(window_load(c)); };
  unsigned win_a, win_b;
  {
    const Win w0 = window_load(0);
    const Win w1 = mw > 64 ? window_load(1) : Win{0u, 0u};
#pragma unroll
    for (int u = 0; u < kQLoads; ++u) {
      const int c = tid + kThreads * u;
      if (c / kChunks < q_rows) s_q[c / kChunks][c % kChunks] = qbuf[u];
    }
    win_a = tile_index(w0);
    win_b = tile_index(w1);
  }
  if constexpr (APPEND) {
    // The step's new token of every stream whose last unit lies in this range goes into the pool
    // here, before any tile is read: the workgroup that reads that unit writes it itself (head
    // tiles of one kv head write the same bytes), so the main loop reads it like any other token.
    // Wave w takes the w-th, (w+4)-th, ... such stream; lane l writes dims 2l and 2l + 1.
    Stream t = cur;
    int k = 0;
    while (t.start < r1) {
      if (t.end <= r1 && k++ % kWaves == wave) {
        const int g = t.gh / a.head_tiles;
        const int p = t.n - 1;  // the new token's position
        const size_t row = (((size_t)t.s * a.num_kv_heads + g) * D) / 2 + lane;
        const bool has = lane < D / 2;
        const unsigned kw = has ? ((const unsigned*)a.new_k)[row] : 0u;
        const unsigned vw = has ? ((const unsigned*)a.new_v)[row] : 0u;
        const unsigned b =
            (unsigned)a.block_tables[(size_t)t.s * a.max_blocks + (p >> (4 + a.sub_shift))];
        wait_vmem();
        if (has) {
          const int tt = p & 15;
          const int d = 2 * lane;
          const size_t tile =
              ((size_t)((b * (unsigned)a.num_kv_heads + (unsigned)g) << (a.sub_shift + 1)) +
               (size_t)((p >> 4) & ((1 << a.sub_shift) - 1))) * (kBlock * D);
          if constexpr (KV8) {  // quantized as reshape_and_cache_fp8 does
            const unsigned kc = e4m3_code(E::widen((unsigned short)kw) * a.k_inv) |
                                e4m3_code(E::widen((unsigned short)(kw >> 16)) * a.k_inv) << 8;
            const unsigned vc = e4m3_code(E::widen((unsigned short)vw) * a.v_inv) |
                                e4m3_code(E::widen((unsigned short)(vw >> 16)) * a.v_inv) << 8;
            unsigned char* kp = (unsigned char*)a.k_pool + tile;
            unsigned char* vp = (unsigned char*)a.v_pool + tile;
            // K8 [d/64][(d/8)%4][token][(d/32)%2][d%8]: dims d, d + 1 are adjacent bytes
            *(unsigned short*)(kp + (size_t)(d / 64) * 1024 + (size_t)(16 * ((d / 8) % 4) + tt) * 16 +
                               ((d / 32) % 2) * 8 + d % 8) = (unsigned short)kc;
#pragma unroll
            for (int e = 0; e < 2; ++e) {  // V8 [d/64][token/4][d%16][(d/16)%4][token%4]
              const int de = d + e;
              vp[(size_t)(de / 64) * 1024 + (size_t)((tt / 4) * 16 + de % 16) * 16 +
                 ((de / 16) % 4) * 4 + tt % 4] = (unsigned char)(vc >> (8 * e));
            }
          } else {
            unsigned short* kp = (unsigned short*)a.k_pool + tile;
            unsigned short* vp = (unsigned short*)a.v_pool + tile;
            // K [d/8][token][d%8]: dims d, d + 1 are one dword
            *(unsigned*)(kp + (size_t)(d / 8) * 128 + (size_t)tt * 8 + d % 8) = kw;
#pragma unroll
            for (int e = 0; e < 2; ++e) {  // V [d/32][token/4][d%16][(d/16)%2][token%4]
              const int de = d + e;
              vp[((((size_t)(de / 32) * 4 + tt / 4) * 16 + de % 16) * 2 + (de / 16) % 2) * 4 +
                 tt % 4] = (unsigned short)(vw >> (16 * e));
            }
          }
        }
      }
      t = stream_after(t);
    }
  }
  wait_vmem();      // the windows (and the new tokens' stores) are complete
  __syncthreads();  // staged q and the new tokens visible to every wave
  int chunk_a = 0;
  auto tile_of = [&](int m) -> unsigned {
    const unsigned w = (m >> 6) == chunk_a ? win_a : win_b;
    return __builtin_amdgcn_readlane(w, m & 63);
  };

  // Q^T operand: lane (hl, kg) holds q[h0 + hl][32c + 8kg .. +8] for each 32-dim chunk c.
  u32x4 qv[NQ];
  auto q_from_lds = [&](int row0, int nvalid) {
#pragma unroll
    for (int c = 0; c < NQ; ++c)
      qv[c] = hl < nvalid ? s_q[row0 + hl][4 * c + kg] : u32x4{0u, 0u, 0u, 0u};
  };
  auto q_from_memory = [&](const Stream& t) {
    const char* qrow = (const char*)a.q + ((size_t)t.s * a.num_q_heads + t.h0 + hl) * D * 2;
#pragma unroll
    for (int c = 0; c < NQ; ++c)
      qv[c] = hl < t.nvalid ? load16(qrow + (32 * c + 8 * kg) * 2) : u32x4{0u, 0u, 0u, 0u};
  };
  q_from_lds(0, cur.nvalid);

  const char* kbase = (const char*)a.k_pool + lane * 16;
  const char* vbase = (const char*)a.v_pool + lane * 16;

  float m_run = -INFINITY;  // reference maximum of head hl (log2 units)
  float l_run = 0.f;        // sum of p over this lane's tokens for head hl
  f32x4 o[NO];
#pragma unroll
  for (int i = 0; i < NO; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Combine layout: 16 lanes per head, kDims consecutive dims per lane.
  const int head = wave * kHeadsPerWave + lane / kLanesPerHead;
  const int d0 = (lane % kLanesPerHead) * kDims;

  // Normalise and store kDims consecutive dims of output row `row`.
  auto store_out = [&](size_t row, const float* acc, float L) {
    const float inv = L > 0.f ? a.v_scale / L : 0.f;  // v_scale: fp8 V pool scale (else 1)
    unsigned short r[kDims];
#pragma unroll
    for (int i = 0; i < kDims; ++i) r[i] = E::store(acc[i] * inv);
    unsigned short* dst = (unsigned short*)a.out + row * D + d0;
    if constexpr (kDims == 8) {
      *(u32x4*)dst = u32x4{r[0] | (unsigned)r[1] << 16, r[2] | (unsigned)r[3] << 16,
                           r[4] | (unsigned)r[5] << 16, r[6] | (unsigned)r[7] << 16};
    } else {
      *(u32x2*)dst = u32x2{r[0] | (unsigned)r[1] << 16, r[2] | (unsigned)r[3] << 16};
    }
  };

  // The four waves' (m, l, O) of the stream just combined in LDS, folded for head `head`, dims
  // d0 .. d0 + kDims (the caller checks head < nvalid).
  auto combine_waves = [&](float& M, float& L, float* acc) {
    M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][head]);
    L = 0.f;
#pragma unroll
    for (int i = 0; i < kDims; ++i) acc[i] = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw_ = sm_m[w][head];
      const float c = mw_ == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw_ - M);  // idle wave
      L += c * sm_l[w][head];
#pragma unroll
      for (int i = 0; i < kDims; ++i) acc[i] += c * sm_o[w][head][d0 + i];
    }
  };
  // A split stream's partial in partial slot `slot` of this workgroup, written through to the
  // device's coherence point (agent-scope stores): the merging workgroup may run on another XCD,
  // behind another L2.
  auto store_partial = [&](int slot, float M, float L, const float* acc) {
    const size_t pidx = ((size_t)wg * 2 + slot) * kMaxGroupTile + head;
    // Element i of lane l (of the head's lanes) at i * kLanesPerHead + l: each store instruction
    // writes whole 64-byte runs of the row.
    float* po = a.ws_o + pidx * D + (lane % kLanesPerHead);
#pragma unroll
    for (int i = 0; i < kDims; ++i)
      __hip_atomic_store(po + i * kLanesPerHead, acc[i], __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    if (lane % kLanesPerHead == 0) {
      __hip_atomic_store(a.ws_ml + pidx * 2, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.ws_ml + pidx * 2 + 1, L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };

  // Split streams of this range: 0 = the one holding r0, 1 = the one holding r1 - 1.
  // Only their start positions stay live through the main loop (scalar registers are the scarce
  // resource there); the merge rebuilds the streams from them. -1: no such stream.
  int split0 = -1, split1 = -1;

  // ---- End of a stream: combine the four waves, then store it or leave its partial. ----
  auto finish_stream = [&]() {
    // The next stream's q: from LDS when staged (no memory access), else from memory, waited for
    // at once so that only ring loads stay outstanding on the common path.
    const Stream nxt = stream_after(cur);
    if (nxt.start < r1) {
      if (staged_left > 0) {
        q_from_lds(next_qrow, nxt.nvalid);
        next_qrow += nxt.nvalid;
        --staged_left;
      } else {
        q_from_memory(nxt);
        wait_vmem();
      }
    }
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
#pragma unroll
      for (int i = 0; i < NO; ++i) sm_o[wave][4 * kg + e][16 * i + hl] = o[i][e];
    }
    if (kg == 0) {
      sm_m[wave][hl] = m_run;
      sm_l[wave][hl] = l_tot;
    }
    m_run = -INFINITY;
    l_run = 0.f;
#pragma unroll
    for (int i = 0; i < NO; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();

    const bool complete = cur.start >= r0 && cur.end <= r1;  // uniform
    const int slot = cur.start <= r0 ? 0 : 1;
    // The stream holding r1 - 1 (slot 1) is always the last one this range finishes, after the
    // main loop: its waves' results stay in LDS for the publish step, which may merge the stream
    // straight from there.
    if (head < cur.nvalid && (complete || slot == 0)) {
      float M, L, acc[kDims];
      combine_waves(M, L, acc);
      if (complete) {
        store_out((size_t)cur.s * a.num_q_heads + cur.h0 + head, acc, L);
      } else {
        store_partial(0, M, L, acc);
      }
    }
    if (!complete) {
      if (slot == 0) {
        split0 = cur.start;
        wait_vmem();  // this wave's share of the partial is at the coherence point
      } else {
        split1 = cur.start;
      }
    }
    if (complete || slot == 0) __syncthreads();  // the combine buffer is free again
    if (!complete && slot == 0 && tid == 0) {
      // Every wave has drained its share: count this part now rather than after the main loop,
      // so that the workgroup finishing the stream's other parts at its range end usually finds
      // them all in and merges at once. A part that completes the count merges after the loop.
      const int wa0 = range_owner(cur.start, nwg, W, odd_w);
      const int np0 = range_owner(cur.end - 1, nwg, W, odd_w) - wa0 + 1;
      const unsigned old = atomicAdd(a.counters + wa0, 1u);
      const int last = old == (unsigned)(np0 - 1);
      if (last) __hip_atomic_store(a.counters + wa0, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last[0] = last;
    }
    cur = nxt;
  };

  // ---- Merge of a split stream by the last of its workgroups to finish. ----
  // Rounds of kMergeRound parts: each lane issues the (m, l) and its output slice of every part
  // of the round before using any of them (one memory round trip per round), then folds the round
  // into a running maximum. Loads are agent-scope: the partials were written through from other
  // XCDs.
  // own: part 0 is this workgroup's, passed in as (own_m, own_l, own_acc) instead of stored.
  auto merge_stream = [&](const Stream& st, bool own, float own_m, float own_l,
                          const float* own_acc) {
    if (head >= st.nvalid) return;  // uniform over each 16-lane head group
    const int wa = range_owner(st.start, nwg, W, odd_w);
    const int np = range_owner(st.end - 1, nwg, W, odd_w) - wa + 1;
    const int slot_a = range_start(wa, nwg, W, odd_w) == st.start ? 0 : 1;
    auto part_idx = [&](int k) {  // partial index of part k (workgroup wa + k)
      return ((size_t)(wa + k) * 2 + (k == 0 ? slot_a : 0)) * kMaxGroupTile + head;
    };
    auto ld = [](const float* p) {
      return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    float M = -INFINITY, L = 0.f;
    float acc[kDims];
#pragma unroll
    for (int i = 0; i < kDims; ++i) acc[i] = 0.f;
    for (int k0 = 0; k0 < np; k0 += kMergeRound) {  // parts in a fixed order
      float mp[kMergeRound], lp[kMergeRound];
      float ov[kMergeRound][kDims];
#pragma unroll
      for (int u = 0; u < kMergeRound; ++u) {
        const size_t pi = part_idx(min(k0 + u, np - 1));  // past the end: reread, weight 0
        mp[u] = ld(a.ws_ml + pi * 2);
        lp[u] = ld(a.ws_ml + pi * 2 + 1);
        const float* po = a.ws_o + pi * D + (lane % kLanesPerHead);
#pragma unroll
        for (int i = 0; i < kDims; ++i) ov[u][i] = ld(po + i * kLanesPerHead);
      }
      if (own && k0 == 0) {  // the same fp32 values the partial would have held
        mp[0] = own_m;
        lp[0] = own_l;
#pragma unroll
        for (int i = 0; i < kDims; ++i) ov[0][i] = own_acc[i];
      }
      float Mr = M;
#pragma unroll
      for (int u = 0; u < kMergeRound; ++u) {
        if (k0 + u < np) Mr = fmaxf(Mr, mp[u]);
      }
      const float rescale = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mr);
      L *= rescale;
#pragma unroll
      for (int i = 0; i < kDims; ++i) acc[i] *= rescale;
#pragma unroll
      for (int u = 0; u < kMergeRound; ++u) {
        const float c = (k0 + u < np && mp[u] != -INFINITY) ? __builtin_amdgcn_exp2f(mp[u] - Mr)
                                                             : 0.f;
        L += c * lp[u];
#pragma unroll
        for (int i = 0; i < kDims; ++i) acc[i] += c * ov[u][i];
      }
      M = Mr;
    }
    store_out((size_t)st.s * a.num_q_heads + st.h0 + head, acc, L);
  };

  // Ring of RING tile buffers: block m + RING - 1 is loading while block m is computed.
  u32x4 kr[RING][NK], vr[RING][NV];
  auto issue = [&](int m, u32x4* kd, u32x4* vd) {
    const unsigned t = tile_of(m);
    const char* kp = kbase + (size_t)t * kTileBytes;
    const char* vp = vbase + (size_t)t * kTileBytes;
#pragma unroll
    for (int c = 0; c < NK; ++c) kd[c] = load16_stream(kp + c * 1024);
#pragma unroll
    for (int c = 0; c < NV; ++c) vd[c] = load16_stream(vp + c * 1024);
  };

  auto process = [&](const u32x4* kc, u32x4* vc, int m) {
    if ((m & 63) == 0 && (m >> 6) != chunk_a) {  // next window of tile ids
      win_a = win_b;
      chunk_a = m >> 6;
      if ((chunk_a + 1) * 64 < mw) {
        win_b = window(chunk_a + 1);
        wait_vmem();
      }
    }
    const int p = r0 + wave + kWaves * m;
    while (p >= cur.end) finish_stream();
    const int j = p - cur.start;  // block of the stream

    // Scores: lane holds S[token 4kg + e][head hl], e = 0..3.
    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
      if constexpr (KV8) {
        // fp8 K: load c/2 holds this lane's 8 dims of chunks c (bytes 0..7) and c+1 (8..15).
        const u32x4 w = kc[c / 2];
        const u32x2 lo = E::from_fp8((c & 1) ? w.z : w.x);
        const u32x2 hi = E::from_fp8((c & 1) ? w.w : w.y);
        sc = E::qk(u32x4{lo.x, lo.y, hi.x, hi.y}, qv[c], sc);
      } else {
        sc = E::qk(kc[c], qv[c], sc);
      }
    }

    const int tb = j * kBlock + 4 * kg;  // token of element e = 0
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = (tb + e < cur.n) ? sc[e] * a.scale_log2 : -INFINITY;
    const float lmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));

    if (__any(lmax > m_run + kLazyRescale)) {
      float gm = fmaxf(lmax, __shfl_xor(lmax, 16));
      gm = fmaxf(gm, __shfl_xor(gm, 32));
      const float m_new = fmaxf(m_run, gm);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ae = __shfl(alpha, 4 * kg + e);  // factor of output row (head 4kg + e)
#pragma unroll
        for (int i = 0; i < NO; ++i) o[i][e] *= ae;
      }
      m_run = m_new;
    }

    float pr[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pr[e] = __builtin_amdgcn_exp2f(x[e] - m_run);
    l_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);
    // P operand(s): one fp16 P against fp16 V; a bf16 high part and residual against bf16 V.
    u32x2 phi, plo = u32x2{0u, 0u};
    if constexpr (kSingleP) {
      phi = EV::round(pr);
    } else {
      E::split(pr, phi, plo);
    }

    // Ragged last block: zero V of dead slots (they may hold anything, NaN included).
    if ((j + 1) * kBlock > cur.n) {
      if constexpr (KV8) {
        // each dword is 4 tokens (one byte each) of one dim
        const unsigned m8 = (tb + 0 < cur.n ? 0x000000FFu : 0u) | (tb + 1 < cur.n ? 0x0000FF00u : 0u) |
                            (tb + 2 < cur.n ? 0x00FF0000u : 0u) | (tb + 3 < cur.n ? 0xFF000000u : 0u);
#pragma unroll
        for (int c = 0; c < NV; ++c) {
          vc[c].x &= m8;
          vc[c].y &= m8;
          vc[c].z &= m8;
          vc[c].w &= m8;
        }
      } else {
        const unsigned m01 = (tb + 0 < cur.n ? 0x0000FFFFu : 0u) | (tb + 1 < cur.n ? 0xFFFF0000u : 0u);
        const unsigned m23 = (tb + 2 < cur.n ? 0x0000FFFFu : 0u) | (tb + 3 < cur.n ? 0xFFFF0000u : 0u);
#pragma unroll
        for (int c = 0; c < NV; ++c) {
          vc[c].x &= m01;
          vc[c].y &= m23;
          vc[c].z &= m01;
          vc[c].w &= m23;
        }
      }
    }

    // O[head][16i + col] += P[head][token] V[token][16i + col]
#pragma unroll
    for (int i = 0; i < NO; ++i) {
      u32x2 vv;
      if constexpr (KV8) {
        // fp8 V: load i/4, dword i%4 holds this lane's 4 tokens of dim 16i + hl.
        const u32x4 w = vc[i / 4];
        vv = EV::from_fp8((i & 3) == 0 ? w.x : (i & 3) == 1 ? w.y : (i & 3) == 2 ? w.z : w.w);
      } else {
        const u32x4 w = vc[i / 2];
        vv = (i & 1) ? u32x2{w.z, w.w} : u32x2{w.x, w.y};
      }
      o[i] = EV::pv(phi, vv, o[i]);
      if constexpr (!kSingleP) o[i] = EV::pv(plo, vv, o[i]);
    }
  };

  // Prologue: blocks 0 .. RING-2 in flight. Issued unconditionally so that every path into the
  // steady loop has the same loads outstanding (a wave with fewer blocks reads tile 0, the
  // window's value past the range, and never uses it).
#pragma unroll
  for (int u = 0; u < RING - 1; ++u) issue(u, kr[u], vr[u]);
  // Steady state: every iteration issues one block and computes one, with no conditions on the
  // loads, so the compiler can count outstanding loads exactly.
  const int steady = mw >= RING - 1 ? (mw - (RING - 1)) / RING * RING : 0;
  for (int j0 = 0; j0 < steady; j0 += RING) {
#pragma unroll
    for (int u = 0; u < RING; ++u) {
      issue(j0 + u + RING - 1, kr[(u + RING - 1) % RING], vr[(u + RING - 1) % RING]);
      process(kr[u], vr[u], j0 + u);
    }
  }
  // Tail: at most 2*RING - 2 blocks; block steady + u sits in slot u % RING.
#pragma unroll
  for (int u = 0; u < 2 * RING - 2; ++u) {
    const int m = steady + u;
    if (m < mw) {
      if (m + RING - 1 < mw) {
        issue(m + RING - 1, kr[(u + RING - 1) % RING], vr[(u + RING - 1) % RING]);
      }
      process(kr[u % RING], vr[u % RING], m);
    }
  }
  // Streams of the range this wave has no further blocks of (every wave joins every combine).
  while (cur.start < r1) finish_stream();

  // ---- Publish the split streams (uniform: every wave saw the same ones). ----
  // A split stream's parts are counted on the arrival counter of its first part's workgroup; the
  // part that brings the count to the number of parts merges them all and resets the counter.
  // Split 0 was counted when its stream ended (s_last[0]); split 1 is counted here.
  const bool has0 = split0 >= 0, has1 = split1 >= 0;
  if (has0 || has1) {
    const Stream st0 = stream_from(has0 ? split0 : split1);
    const Stream st1 = stream_from(has1 ? split1 : split0);
    const int np1 = range_owner(st1.end - 1, nwg, W, odd_w) - wg + 1;  // st1 starts in this range
    // Split 1's own part, folded once from the combine buffer: both ways of finishing it below
    // use these very values, so the result cannot depend on which workgroup arrives last.
    float m1 = 0.f, l1 = 0.f, acc1[kDims];
#pragma unroll
    for (int i = 0; i < kDims; ++i) acc1[i] = 0.f;
    if (has1 && head < st1.nvalid) combine_waves(m1, l1, acc1);
    __syncthreads();  // s_last[0] (set when split 0 ended) is visible
    if (tid == 1 && has1) {
      // Split 1 begins here, so its counter is this workgroup's. When every other part has
      // already arrived, this workgroup is the last: it merges at once, taking its own part from
      // the combine buffer, and skips storing, draining and counting that part.
      const unsigned seen =
          __hip_atomic_load(a.counters + wg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int fast = seen == (unsigned)(np1 - 1);
      if (fast) __hip_atomic_store(a.counters + wg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last[1] = fast;
    }
    __syncthreads();
    if (has0 && s_last[0]) merge_stream(st0, false, 0.f, 0.f, acc1);
    if (has1) {
      if (s_last[1]) {
        merge_stream(st1, true, m1, l1, acc1);
      } else {
        if (head < st1.nvalid) store_partial(1, m1, l1, acc1);
        wait_vmem();
        __syncthreads();
        if (tid == 1) {
          const unsigned old = atomicAdd(a.counters + wg, 1u);
          const int last = old == (unsigned)(np1 - 1);
          if (last)
            __hip_atomic_store(a.counters + wg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          s_last[1] = last;
        }
        __syncthreads();
        if (s_last[1]) merge_stream(st1, false, 0.f, 0.f, acc1);
      }
    }
  }
}

template <int D, bool BF16, bool KV8, bool APPEND>
hipError_t launch_typed(const DecodeLaunch& a, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((paged_decode_kernel<D, BF16, KV8, APPEND, kRing<D>>),
                     dim3((unsigned)grid), dim3(64 * kWaves), 0, stream, a);
  return hipGetLastError();
}

template <int D, bool KV8, bool APPEND>
hipError_t launch_dtype(const DecodeLaunch& a, int grid, bool bf16, hipStream_t stream) {
  return bf16 ? launch_typed<D, true, KV8, APPEND>(a, grid, stream)
              : launch_typed<D, false, KV8, APPEND>(a, grid, stream);
}

template <int D, bool APPEND>
hipError_t launch_kv(const DecodeLaunch& a, int grid, bool bf16, bool kv_fp8, hipStream_t stream) {
  return kv_fp8 ? launch_dtype<D, true, APPEND>(a, grid, bf16, stream)
                : launch_dtype<D, false, APPEND>(a, grid, bf16, stream);
}

}  // namespace

hipError_t launch_decode(const DecodeLaunch& a, int grid, int head_dim, bool bf16, bool kv_fp8,
                         bool append, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  if (head_dim == 128) {
    return append ? launch_kv<128, true>(a, grid, bf16, kv_fp8, stream)
                  : launch_kv<128, false>(a, grid, bf16, kv_fp8, stream);
  }
  return append ? launch_kv<64, true>(a, grid, bf16, kv_fp8, stream)
                : launch_kv<64, false>(a, grid, bf16, kv_fp8, stream);
}

}  // namespace pkv
