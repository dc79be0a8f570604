// Internal declarations shared by the HIP translation units of libpagedkv (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

constexpr int kBlock = 16;          // tokens per sub-tile: the decode's unit of work (a
                                    // physical block holds 1 or 2 sub-tiles: block size 16 or 32)
constexpr int kMaxGroupTile = 16;   // query heads per wave (matrix-core N dimension)
constexpr int kWaves = 4;           // wavefronts per decode workgroup
constexpr int kMaxSeqs = 2048;      // sequences one decode launch plans for (LDS prefix sums)
constexpr int kWorkgroupsPerCU = 2; // resident decode workgroups per compute unit

// OCP E4M3 code of an fp32 value: round to nearest even, saturating at +-448, NaN kept (with its
// sign), sign kept for zero. Integer arithmetic on the fp32 bits, so every device gives the same
// code.
__device__ __forceinline__ unsigned e4m3_code(float y) {
  const unsigned bits = __float_as_uint(y);
  const unsigned sign = (bits >> 24) & 0x80u;
  const unsigned a = bits & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;  // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu; // |y| >= 448 (and infinity): saturate
  const int e = (int)(a >> 23) - 127;        // exponent of |y| (fp32 denormals: -127)
  if (e < -6) {
    // Below the smallest normal 2^-6: code = |y| * 2^9 rounded, i.e. the 24-bit significand
    // shifted right by 14 - e bits (a result of 8 is the smallest normal, code 0x08).
    const int sh = 14 - e;
    if (sh >= 32) return sign;
    const unsigned sig = (a & 0x7FFFFFu) | 0x800000u;
    unsigned q = sig >> sh;
    const unsigned rem = sig & ((1u << sh) - 1u);
    const unsigned half = 1u << (sh - 1);
    q += (rem > half || (rem == half && (q & 1u))) ? 1u : 0u;
    return sign | q;
  }
  // Normal: 3 mantissa bits from 23, exponent field e + 7.
  const unsigned m = a & 0x7FFFFFu;
  unsigned q = m >> 20;
  const unsigned rem = m & 0xFFFFFu;
  q += (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) ? 1u : 0u;
  unsigned ef = (unsigned)(e + 7);
  if (q == 8u) {
    q = 0u;
    ++ef;
  }
  return sign | (ef << 3) | q;
}

// ---- Decode workgroup ranges ----
// The decode cuts its flattened block positions [0, W) into nwg contiguous ranges, one per
// workgroup. Workgroups are dispatched round-robin over the 8 XCDs of MI355X (XCD = blockIdx % 8
// when the GPU runs as one partition, SPX), each XCD with its own L2. When nwg is a multiple of
// 8 the ranges are handed out in XCD blocks: range r runs on workgroup (r % P) * 8 + r / P,
// P = nwg / 8, so XCD x executes the P consecutive ranges [x P, (x + 1) P) -- one contiguous
// stretch of positions, and streams that read the same blocks (a shared prompt prefix) are read
// through one L2. Otherwise range r runs on workgroup r.
// The odd-numbered XCDs stream measurably slower (about 9% on the 70B-shaped decode, on every
// board measured), so a range's share is proportional to a weight: kEvenWeight for ranges of an
// even XCD block, odd_weight for an odd one (with one block, every range weighs kEvenWeight).
// Range r covers [range_start(r), range_start(r + 1)).
constexpr int kEvenWeight = 1024;

// XCD blocks the ranges of an nwg-workgroup launch are grouped in: 8, or 1 (no grouping).
__host__ __device__ inline int range_blocks(int nwg) { return nwg % 8 == 0 ? 8 : 1; }

// The range workgroup w executes, and its inverse.
__host__ __device__ inline int range_of_workgroup(int w, int nwg) {
  const int nx = range_blocks(nwg), per = nwg / nx;
  return (w % nx) * per + w / nx;
}
__host__ __device__ inline int workgroup_of_range(int r, int nwg) {
  const int nx = range_blocks(nwg), per = nwg / nx;
  return (r % per) * nx + r / per;
}

// C(r): sum of the weights of ranges 0 .. r - 1 (r in [0, nwg]).
__host__ __device__ inline long long range_cum_weight(int r, int nwg, int odd_weight) {
  const int nx = range_blocks(nwg), per = nwg / nx;
  const int x = r / per;
  const int i = r - x * per;
  const long long w = nx == 1 ? kEvenWeight : (x & 1) ? odd_weight : kEvenWeight;
  const long long ow = nx == 1 ? kEvenWeight : odd_weight;
  return (long long)per * ((long long)((x + 1) / 2) * kEvenWeight + (long long)(x / 2) * ow) +
         (long long)i * w;
}

__host__ __device__ inline int range_start(int r, int nwg, int W, int odd_weight) {
  return (int)((long long)W * range_cum_weight(r, nwg, odd_weight) /
               range_cum_weight(nwg, nwg, odd_weight));
}

// The range holding position p (0 <= p < W): the last r < nwg with range_start(r) <= p, i.e. with
// C(r) <= ceil((p + 1) C(nwg) / W) - 1: first the XCD block, then the range inside it.
__host__ __device__ inline int range_owner(int p, int nwg, int W, int odd_weight) {
  const long long x = ((long long)(p + 1) * range_cum_weight(nwg, nwg, odd_weight) - 1) / W;
  const int nx = range_blocks(nwg), per = nwg / nx;
  int b = nx - 1;
  while (b > 0 && range_cum_weight(b * per, nwg, odd_weight) > x) --b;
  const long long w = nx == 1 ? kEvenWeight : (b & 1) ? odd_weight : kEvenWeight;
  long long i = (x - range_cum_weight(b * per, nwg, odd_weight)) / w;
  if (i > per - 1) i = per - 1;
  const long long r = (long long)b * per + i;
  return (int)(r < nwg - 1 ? r : nwg - 1);
}

// How a launch of `grid` workgroups cuts W positions: the workgroups that get a range (the rest
// exit) and the weight of odd-XCD ranges. L is the units of every sequence when all sequences have
// the same number, else 0.
//  * Weighted ranges only when they can help and cannot hurt: every range must keep at least one
//    position (W >= 2 nwg, weights in [kEvenWeight / 2, kEvenWeight]), since the split-stream
//    bookkeeping needs non-empty ranges; and the equal split must not already fall on stream
//    boundaries (all streams of length L with W / nwg a whole number of streams), where it splits
//    no stream and any weighting would add a merge to every workgroup.
//  * may_halve (the host chose a full grid and there are at most as many streams as workgroups):
//    when the equal split would cut streams, one workgroup per compute unit (the first half of
//    the grid) cuts half as many.
struct RangePlan {
  int nwg;       // workgroups with a range: 0 .. nwg - 1
  int odd_w;     // range weight on odd XCDs (kEvenWeight: equal ranges)
  bool aligned;  // equal ranges of W / nwg positions, each a whole number of streams
};

__host__ __device__ inline RangePlan plan_ranges(int W, int L, int grid, bool may_halve,
                                                 int odd_weight) {
  int nwg = grid < W ? grid : W;
  auto aligned_for = [&](int n) { return L > 0 && W % n == 0 && (W / n) % L == 0; };
  bool aligned = nwg > 0 && aligned_for(nwg);
  if (may_halve && !aligned && nwg >= 2) {
    nwg /= 2;
    aligned = aligned_for(nwg);
  }
  return RangePlan{nwg, W >= 2 * nwg && !aligned ? odd_weight : kEvenWeight, aligned};
}

struct DecodeLaunch {
  void* out;
  const void* q;
  const void* k_pool;   // K and V planes of one layer: the tiles of (block b, kv head g) start
  const void* v_pool;   // 2 * (b * num_kv_heads + g) tiles into each
  const int32_t* block_tables;
  const int32_t* context_lens;
  unsigned* counters;   // [grid] arrival counts of split streams; zero between launches
  float* ws_o;          // [grid][2][16][D] unnormalised partial outputs of split streams
  float* ws_ml;         // [grid][2][16][2] (reference max in log2 units, row sum)
  float scale_log2;     // scale * log2(e) (times the K pool scale for fp8 pools)
  float v_scale;        // V pool scale for fp8 pools, else 1
  int num_seqs;
  int num_q_heads;
  int num_kv_heads;
  int group;            // num_q_heads / num_kv_heads
  int head_tiles;       // ceil(group / 16)
  int max_blocks;       // block table row length
  int max_tokens;       // max_blocks * block_size: context lengths are clamped to it
  int sub_shift;        // log2(block_size / 16): sub-tiles per physical block = 1 << sub_shift
  // Fused append (the step's new token of each sequence, at position context_len - 1, taken from
  // these rows instead of the pool and written into the pool): [num_seqs][num_kv_heads][D].
  const void* new_k;
  const void* new_v;
  float k_inv;          // fp8 pools: 1 / k_scale and 1 / v_scale (the new token's quantization)
  float v_inv;
  int odd_weight;       // range weight of workgroups on odd XCDs (even ones: kEvenWeight)
  int may_halve;        // the library chose a full grid and there are at most as many streams
                        // as workgroups: the kernel may use half of them (plan_ranges)
};

// Launch the decode kernel on `grid` workgroups (append: the fused variant that takes each
// sequence's newest token from new_k / new_v). Returns a hipError_t.
hipError_t launch_decode(const DecodeLaunch& a, int grid, int head_dim, bool bf16, bool kv_fp8,
                         bool append, hipStream_t stream);

// reshape_and_cache into fp8 (E4M3) pools: code = e4m3(fl32(x * inv_scale)) per element.
hipError_t launch_reshape_and_cache_fp8(const void* key, const void* value, void* k_pool,
                                        void* v_pool, const int64_t* slot_mapping, int num_tokens,
                                        int num_kv_heads, int head_dim, int block_size,
                                        int num_blocks, bool src_bf16, float k_inv_scale,
                                        float v_inv_scale, hipStream_t stream);

// One whole-block copy launch: pair i copies block src_ids[i] of the source pool to block
// dst_ids[i] of the destination pool in every layer. A block's region in one layer (the K and V
// tiles of all its kv heads) is contiguous. Addresses are device-visible (a pinned host pool is
// passed by its device address).
struct BlockCopy {
  const char* src;        // pool bases (layer 0, block 0)
  char* dst;
  size_t src_layer_bytes;
  size_t dst_layer_bytes;
  size_t block_bytes;     // one layer's region of one block: num_kv_heads * 2 * block_size * D * elem
  const int32_t* src_ids;
  const int32_t* dst_ids;
  int src_blocks;         // ids outside [0, src_blocks) / [0, dst_blocks) are skipped
  int dst_blocks;
};

hipError_t launch_block_copy(const BlockCopy& c, int num_layers, int num_pairs,
                             hipStream_t stream);

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_pool, void* v_pool,
                                    const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                                    int head_dim, int block_size, int num_blocks,
                                    hipStream_t stream);

}  // namespace pkv
