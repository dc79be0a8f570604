// reshape_and_cache: scatter one step's new keys/values into their pool slots.
//
// Boundary allocation ("PagedAttention and KV Cache Management" (blog.sejan.dev), section "How
// Block Paging Operates During Generation") gives every new token a slot = block * 16 + t; this
// kernel writes the token's K and V rows for every kv head into that slot of the pool's tiles.
// One thread moves eight consecutive dims (16 bytes) of one (token, kv head): the K tile keeps
// those eight dims contiguous, so K is one 16-byte store; the V tile keeps four consecutive
// tokens of one dim together, so V is eight 2-byte stores.

#include "pkv_internal.h"

namespace pkv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int D>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const unsigned short* __restrict__ key, const unsigned short* __restrict__ value,
    unsigned short* __restrict__ k_pool, unsigned short* __restrict__ v_pool,
    const int64_t* __restrict__ slot_mapping, int num_tokens, int num_kv_heads, int block_size) {
  constexpr int kChunks = D / 8;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long total = (long)num_tokens * num_kv_heads * kChunks;
  if (gid >= total) return;
  const int c = (int)(gid % kChunks);
  const long r = gid / kChunks;
  const int h = (int)(r % num_kv_heads);
  const long i = r / num_kv_heads;
  const int64_t slot = slot_mapping[i];
  if (slot < 0) return;
  const int64_t b = slot / block_size;
  const int tb = (int)(slot % block_size);
  const int t = tb % kBlock;  // token within its 16-token sub-tile
  // tile of (block, kv head), then the sub-tile holding the token
  const size_t tile = ((size_t)b * num_kv_heads + h) * (size_t)block_size * D +
                      (size_t)(tb / kBlock) * (kBlock * D);
  const size_t src = ((size_t)i * num_kv_heads + h) * D + 8 * c;

  *(u32x4*)(k_pool + tile + c * 128 + t * 8) = *(const u32x4*)(key + src);

  const u32x4 w = *(const u32x4*)(value + src);
  const unsigned words[4] = {w.x, w.y, w.z, w.w};
  // dims 8c .. 8c+7 share d/32, d/16 (their 16-dim half) and run through d%16 = 8(c%2) + e.
  const int d0 = 8 * c;
  const size_t base = tile + ((((size_t)(d0 / 32) * 4 + t / 4) * 16 + (d0 % 16)) * 2 +
                              (d0 / 16) % 2) * 4 + t % 4;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const unsigned short bits = (unsigned short)(words[e / 2] >> (16 * (e % 2)));
    v_pool[base + (size_t)e * 8] = bits;  // d%16 + 1 -> +2*4 elements
  }
}

// copy_blocks: for every pair i and layer L, the K and V regions of block src[i] (all kv heads,
// B * D elements each) are copied to block dst[i]. One thread moves 16 bytes; the grid is
// (16-byte chunks of a block region / 256, pairs, layers * 2 (K, V)), so consecutive workgroups
// stream consecutive 4 KiB of one region. Pure streaming copy. (Measured: one workgroup per
// region with 8 loads in flight per thread was 15% slower.)
__global__ __launch_bounds__(256) void copy_blocks_kernel(char* __restrict__ k_pool,
                                                         char* __restrict__ v_pool,
                                                         size_t layer_bytes, size_t block_bytes,
                                                         const int32_t* __restrict__ src,
                                                         const int32_t* __restrict__ dst) {
  const size_t chunk = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (chunk * 16 >= block_bytes) return;
  const int i = blockIdx.y;
  const int layer = blockIdx.z >> 1;
  char* pool = (blockIdx.z & 1) ? v_pool : k_pool;
  char* base = pool + (size_t)layer * layer_bytes + chunk * 16;
  const u32x4 w = __builtin_nontemporal_load((const u32x4*)(base + (size_t)src[i] * block_bytes));
  __builtin_nontemporal_store(w, (u32x4*)(base + (size_t)dst[i] * block_bytes));
}

}  // namespace

hipError_t launch_copy_blocks(void* k_pool, void* v_pool, size_t layer_bytes, size_t block_bytes,
                              int num_layers, const int32_t* src, const int32_t* dst,
                              int num_copies, hipStream_t stream) {
  if (num_copies == 0) return hipSuccess;
  const size_t chunks = block_bytes / 16;
  const dim3 grid((unsigned)((chunks + 255) / 256), (unsigned)num_copies, (unsigned)(2 * num_layers));
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(256), 0, stream, (char*)k_pool, (char*)v_pool,
                     layer_bytes, block_bytes, src, dst);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_pool, void* v_pool,
                                    const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                                    int head_dim, int block_size, hipStream_t stream) {
  const long total = (long)num_tokens * num_kv_heads * (head_dim / 8);
  if (total == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total + 255) / 256);
  const auto* k = (const unsigned short*)key;
  const auto* v = (const unsigned short*)value;
  auto* kp = (unsigned short*)k_pool;
  auto* vp = (unsigned short*)v_pool;
  if (head_dim == 128) {
    hipLaunchKernelGGL(reshape_and_cache_kernel<128>, dim3(blocks), dim3(256), 0, stream, k, v, kp,
                       vp, slot_mapping, num_tokens, num_kv_heads, block_size);
  } else {
    hipLaunchKernelGGL(reshape_and_cache_kernel<64>, dim3(blocks), dim3(256), 0, stream, k, v, kp,
                       vp, slot_mapping, num_tokens, num_kv_heads, block_size);
  }
  return hipGetLastError();
}

}  // namespace pkv
