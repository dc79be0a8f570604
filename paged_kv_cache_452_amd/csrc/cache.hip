// reshape_and_cache: scatter one step's new keys/values into their pool slots.
//
// Boundary allocation ("PagedAttention and KV Cache Management" (blog.sejan.dev), section "How
// Block Paging Operates During Generation") gives every new token a slot = block * 16 + t; this
// kernel writes the token's K and V rows for every kv head into that slot of the pool's tiles.
// One thread moves eight consecutive dims (16 bytes) of one (token, kv head): the K tile keeps
// those eight dims contiguous, so K is one 16-byte store; the V tile keeps four consecutive
// tokens of one dim together, so V is eight 2-byte stores. A wavefront takes consecutive tokens
// of one kv head, so the stores of a prompt's consecutive tokens land side by side and merge.

#include "pkv_internal.h"
#include "pkv_link.h"

namespace pkv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Tokens per wavefront of the scatter kernels: 64 lanes over a token's D / 8 chunks of 16 bytes.
// Consecutive tokens of one wavefront that fill consecutive slots (a prompt's do) then write
// adjacent bytes in one store instruction, which the memory pipeline merges: their K chunks are
// 16 bytes apart and their V values 2 bytes apart (1 byte in fp8 pools).
template <int D>
constexpr int scatter_tokens() {
  return 64 / (D / 8);
}

// Threads of a scatter launch: whole wavefronts of scatter_tokens<D>() tokens per kv head.
template <int D>
long scatter_threads(int num_tokens, int num_kv_heads) {
  return (long)((num_tokens + scatter_tokens<D>() - 1) / scatter_tokens<D>()) * num_kv_heads * 64;
}

template <int D>
__global__ __launch_bounds__(256) void reshape_and_cache_kernel(
    const unsigned short* __restrict__ key, const unsigned short* __restrict__ value,
    unsigned short* __restrict__ k_pool, unsigned short* __restrict__ v_pool,
    const int64_t* __restrict__ slot_mapping, int num_tokens, int num_kv_heads, int block_size,
    int64_t num_slots) {
  constexpr int kChunks = D / 8;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  // a wavefront: one kv head, scatter_tokens<D>() consecutive tokens, each token's 16-byte chunks
  // on consecutive lanes
  const int c = (int)(gid % kChunks);
  const long i = (gid / 64 / num_kv_heads) * scatter_tokens<D>() + (gid % 64) / kChunks;
  const int h = (int)(gid / 64 % num_kv_heads);
  if (i >= num_tokens) return;
  const int64_t slot = slot_mapping[i];
  if (slot < 0 || slot >= num_slots) return;  // skipped: negative or past the pool
  const int64_t b = slot / block_size;
  const int tb = (int)(slot % block_size);
  const int t = tb % kBlock;  // token within its 16-token sub-tile
  // tile of (block, kv head) in its plane (K and V tiles alternate: a stride of two tiles), then
  // the sub-tile holding the token
  const size_t tile = ((size_t)b * num_kv_heads + h) * (size_t)(2 * block_size) * D +
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

// reshape_and_cache into fp8 pools: one thread quantizes eight consecutive dims of one (token,
// kv head): K is one 8-byte store (the fp8 K tile keeps those eight dims contiguous), V eight
// byte stores (the fp8 V tile keeps four consecutive tokens of a dim together).
template <int D, bool BF16>
__global__ __launch_bounds__(256) void reshape_and_cache_fp8_kernel(
    const unsigned short* __restrict__ key, const unsigned short* __restrict__ value,
    unsigned char* __restrict__ k_pool, unsigned char* __restrict__ v_pool,
    const int64_t* __restrict__ slot_mapping, int num_tokens, int num_kv_heads, int block_size,
    int64_t num_slots, float k_inv, float v_inv) {
  constexpr int kChunks = D / 8;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  // a wavefront: one kv head, scatter_tokens<D>() consecutive tokens, each token's 16-byte chunks
  // on consecutive lanes
  const int c = (int)(gid % kChunks);
  const long i = (gid / 64 / num_kv_heads) * scatter_tokens<D>() + (gid % 64) / kChunks;
  const int h = (int)(gid / 64 % num_kv_heads);
  if (i >= num_tokens) return;
  const int64_t slot = slot_mapping[i];
  if (slot < 0 || slot >= num_slots) return;  // skipped: negative or past the pool
  const int64_t b = slot / block_size;
  const int tb = (int)(slot % block_size);
  const int t = tb % kBlock;
  const size_t tile = ((size_t)b * num_kv_heads + h) * (size_t)(2 * block_size) * D +
                      (size_t)(tb / kBlock) * (kBlock * D);
  const size_t src = ((size_t)i * num_kv_heads + h) * D + 8 * c;
  const u32x4 kw = *(const u32x4*)(key + src);
  const u32x4 vw = *(const u32x4*)(value + src);
  const unsigned kwords[4] = {kw.x, kw.y, kw.z, kw.w};
  const unsigned vwords[4] = {vw.x, vw.y, vw.z, vw.w};
  auto widen = [](unsigned short bits) -> float {
    if constexpr (BF16) {
      return __uint_as_float((unsigned)bits << 16);
    } else {
      return (float)__builtin_bit_cast(_Float16, bits);
    }
  };
  const int d0 = 8 * c;
  unsigned kc[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const unsigned short kb = (unsigned short)(kwords[e / 2] >> (16 * (e % 2)));
    kc[e / 4] |= e4m3_code(widen(kb) * k_inv) << (8 * (e % 4));
  }
  // K: [d/64][(d/8)%4][token][(d/32)%2][d%8] -> dims d0..d0+7 are 8 contiguous bytes
  const size_t koff = tile + (size_t)(d0 / 64) * 1024 + (size_t)(16 * ((d0 / 8) % 4) + t) * 16 +
                      (size_t)((d0 / 32) % 2) * 8;
  *(u32x2*)(k_pool + koff) = u32x2{kc[0], kc[1]};
  // V: [d/64][token/4][d%16][(d/16)%4][token%4]
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int d = d0 + e;
    const unsigned short vb = (unsigned short)(vwords[e / 2] >> (16 * (e % 2)));
    v_pool[tile + (size_t)(d / 64) * 1024 + (size_t)((t / 4) * 16 + d % 16) * 16 +
           (size_t)((d / 16) % 4) * 4 + t % 4] = (unsigned char)e4m3_code(widen(vb) * v_inv);
  }
}

// Whole-block copies within the device pool (copy-on-write; swapping to and from host memory uses
// block_copy_link_kernel below). For pair i and layer L, the region of block src[i] (the K and V
// tiles of all kv heads: block_bytes, contiguous) is copied to block dst[i]. One thread moves 16
// bytes; the grid is (16-byte chunks of a region / 256, pairs, layers), so consecutive workgroups
// stream consecutive 4 KiB of one region. A pair with an id outside its pool is skipped. Pure
// streaming copy. (Measured on device pools: one workgroup per region with 8 loads in flight per
// thread was 15% slower.)
__global__ __launch_bounds__(256) void block_copy_kernel(BlockCopy c) {
  const size_t chunk = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (chunk * 16 >= c.block_bytes) return;
  const int i = blockIdx.y;
  const int s = c.src_ids[i];
  const int d = c.dst_ids[i];
  if (s < 0 || s >= c.src_blocks || d < 0 || d >= c.dst_blocks) return;
  const int layer = blockIdx.z;
  const char* src = c.src + (size_t)layer * c.src_layer_bytes + (size_t)s * c.block_bytes + chunk * 16;
  char* dst = c.dst + (size_t)layer * c.dst_layer_bytes + (size_t)d * c.block_bytes + chunk * 16;
  const u32x4 w = __builtin_nontemporal_load((const u32x4*)src);
  __builtin_nontemporal_store(w, (u32x4*)dst);
}

// The same copies over the host link (swapping), from a small fixed grid. The link moves about
// 55 GB/s, far less than the compute units can issue, so kLinkWorkgroups workgroups with
// kLinkUnroll 16-byte loads in flight per thread keep it busy (measured: swap in 57.4 GB/s and
// swap out 54.9 GB/s, against 54.7 and 53.8 GB/s with one workgroup per 4 KiB as above). Fewer
// workgroups do not spare a decode running beside the swap: compute-unit accesses to host memory
// slow such a decode by ~80% whatever the grid, which the copy-engine path (swap_blocks_dma)
// avoids. Each workgroup takes whole regions in turn: region r is pair r % num_pairs of layer
// r / num_pairs. The block ids of its next region, which may sit in pinned host memory (a round
// trip over the link), are read while the current region is copied.
__global__ __launch_bounds__(256) void block_copy_link_kernel(BlockCopy c, int num_layers,
                                                              int num_pairs) {
  const long regions = (long)num_layers * num_pairs;
  const int chunks = (int)(c.block_bytes / 16);
  long r = blockIdx.x;
  if (r >= regions) return;
  int s = c.src_ids[r % num_pairs];
  int d = c.dst_ids[r % num_pairs];
  for (; r < regions; r += gridDim.x) {
    const long rn = r + gridDim.x;
    int sn = 0, dn = 0;
    if (rn < regions) {
      sn = c.src_ids[rn % num_pairs];
      dn = c.dst_ids[rn % num_pairs];
    }
    if (s >= 0 && s < c.src_blocks && d >= 0 && d < c.dst_blocks) {
      const size_t layer = (size_t)(r / num_pairs);
      const char* src = c.src + layer * c.src_layer_bytes + (size_t)s * c.block_bytes;
      char* dst = c.dst + layer * c.dst_layer_bytes + (size_t)d * c.block_bytes;
      for (int k0 = threadIdx.x; k0 < chunks; k0 += 256 * kLinkUnroll) {
        u32x4 w[kLinkUnroll];
#pragma unroll
        for (int u = 0; u < kLinkUnroll; ++u) {
          const int k = k0 + 256 * u;
          if (k < chunks) w[u] = __builtin_nontemporal_load((const u32x4*)(src + (size_t)k * 16));
        }
#pragma unroll
        for (int u = 0; u < kLinkUnroll; ++u) {
          const int k = k0 + 256 * u;
          if (k < chunks) __builtin_nontemporal_store(w[u], (u32x4*)(dst + (size_t)k * 16));
        }
      }
    }
    s = sn;
    d = dn;
  }
}

}  // namespace

hipError_t launch_block_copy_link(const BlockCopy& c, int num_layers, int num_pairs,
                                  hipStream_t stream) {
  if (num_pairs == 0) return hipSuccess;
  const long regions = (long)num_layers * num_pairs;
  const unsigned grid = (unsigned)(regions < kLinkWorkgroups ? regions : kLinkWorkgroups);
  hipLaunchKernelGGL(block_copy_link_kernel, dim3(grid), dim3(256), 0, stream, c, num_layers,
                     num_pairs);
  return hipGetLastError();
}

hipError_t launch_block_copy(const BlockCopy& c, int num_layers, int num_pairs,
                             hipStream_t stream) {
  if (num_pairs == 0) return hipSuccess;
  const size_t chunks = c.block_bytes / 16;
  const dim3 grid((unsigned)((chunks + 255) / 256), (unsigned)num_pairs, (unsigned)num_layers);
  hipLaunchKernelGGL(block_copy_kernel, grid, dim3(256), 0, stream, c);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache_fp8(const void* key, const void* value, void* k_pool,
                                        void* v_pool, const int64_t* slot_mapping, int num_tokens,
                                        int num_kv_heads, int head_dim, int block_size,
                                        int num_blocks, bool src_bf16, float k_inv_scale,
                                        float v_inv_scale, hipStream_t stream) {
  const int64_t num_slots = (int64_t)num_blocks * block_size;
  if (num_tokens == 0 || num_kv_heads == 0) return hipSuccess;
  const long total = head_dim == 128 ? scatter_threads<128>(num_tokens, num_kv_heads)
                                     : scatter_threads<64>(num_tokens, num_kv_heads);
  const unsigned blocks = (unsigned)((total + 255) / 256);
  const auto* k = (const unsigned short*)key;
  const auto* v = (const unsigned short*)value;
  auto* kp = (unsigned char*)k_pool;
  auto* vp = (unsigned char*)v_pool;
#define PKV_RC8(DD, BB)                                                                          \
  hipLaunchKernelGGL((reshape_and_cache_fp8_kernel<DD, BB>), dim3(blocks), dim3(256), 0, stream, \
                     k, v, kp, vp, slot_mapping, num_tokens, num_kv_heads, block_size,           \
                     num_slots, k_inv_scale, v_inv_scale)
  if (head_dim == 128) {
    if (src_bf16) PKV_RC8(128, true); else PKV_RC8(128, false);
  } else {
    if (src_bf16) PKV_RC8(64, true); else PKV_RC8(64, false);
  }
#undef PKV_RC8
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_pool, void* v_pool,
                                    const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                                    int head_dim, int block_size, int num_blocks,
                                    hipStream_t stream) {
  const int64_t num_slots = (int64_t)num_blocks * block_size;
  if (num_tokens == 0 || num_kv_heads == 0) return hipSuccess;
  const long total = head_dim == 128 ? scatter_threads<128>(num_tokens, num_kv_heads)
                                     : scatter_threads<64>(num_tokens, num_kv_heads);
  const unsigned blocks = (unsigned)((total + 255) / 256);
  const auto* k = (const unsigned short*)key;
  const auto* v = (const unsigned short*)value;
  auto* kp = (unsigned short*)k_pool;
  auto* vp = (unsigned short*)v_pool;
  if (head_dim == 128) {
    hipLaunchKernelGGL(reshape_and_cache_kernel<128>, dim3(blocks), dim3(256), 0, stream, k, v, kp,
                       vp, slot_mapping, num_tokens, num_kv_heads, block_size, num_slots);
  } else {
    hipLaunchKernelGGL(reshape_and_cache_kernel<64>, dim3(blocks), dim3(256), 0, stream, k, v, kp,
                       vp, slot_mapping, num_tokens, num_kv_heads, block_size, num_slots);
  }
  return hipGetLastError();
}

}  // namespace pkv
