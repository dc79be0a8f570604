// Internal declarations shared by the HIP translation units of libpagedkv (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

constexpr int kBlock = 16;          // tokens per physical block this build supports
constexpr int kMaxGroupTile = 16;   // query heads per wave (matrix-core N dimension)
constexpr int kWaves = 4;           // wavefronts per decode workgroup
constexpr int kWaveBlocks = 64;     // blocks one wavefront handles at most (ids in one VGPR)
constexpr int kMaxPartBlocks = kWaves * kWaveBlocks;  // blocks per workgroup (partition)

struct DecodeLaunch {
  void* out;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_o;          // [S][Hq][max_parts][D] unnormalised partial outputs
  float* ws_ml;         // [S][Hq][max_parts][2] (running max in log2 units, row sum)
  float scale_log2;     // scale * log2(e)
  int num_seqs;
  int num_q_heads;
  int num_kv_heads;
  int group;            // num_q_heads / num_kv_heads
  int head_tiles;       // ceil(group / 16)
  int max_blocks;       // block table row length
  int part_blocks;      // most blocks of one partition (<= kMaxPartBlocks); a sequence of nb
                        // blocks has ceil(nb / part_blocks) partitions of near-equal length
  int max_parts;        // partitions of the longest allowed sequence
};

// Launch the decode kernel (and the merge when max_parts > 1). Returns a hipError_t.
hipError_t launch_decode(const DecodeLaunch& a, int head_dim, bool bf16, hipStream_t stream);

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_pool, void* v_pool,
                                    const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                                    int head_dim, hipStream_t stream);

}  // namespace pkv
