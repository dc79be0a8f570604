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

struct DecodeLaunch {
  void* out;
  const void* q;
  const void* k_pool;
  const void* v_pool;
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
};

// Launch the decode kernel on `grid` workgroups. Returns a hipError_t.
hipError_t launch_decode(const DecodeLaunch& a, int grid, int head_dim, bool bf16, bool kv_fp8,
                         hipStream_t stream);

// reshape_and_cache into fp8 (E4M3) pools: code = e4m3(fl32(x * inv_scale)) per element.
hipError_t launch_reshape_and_cache_fp8(const void* key, const void* value, void* k_pool,
                                        void* v_pool, const int64_t* slot_mapping, int num_tokens,
                                        int num_kv_heads, int head_dim, int block_size,
                                        int num_blocks, bool src_bf16, float k_inv_scale,
                                        float v_inv_scale, hipStream_t stream);

// Copy the K and V regions of blocks src[i] -> dst[i] in every layer (device arrays).
// One whole-block copy launch: pair i copies block src_ids[i] of the source pool to block
// dst_ids[i] of the destination pool, K and V of every layer. Addresses are device-visible (a
// pinned host pool is passed by its device address).
struct BlockCopy {
  const char* src_k;
  const char* src_v;
  char* dst_k;
  char* dst_v;
  size_t src_layer_bytes;
  size_t dst_layer_bytes;
  size_t block_bytes;     // one layer's region of one block: num_kv_heads * block_size * D * elem
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
