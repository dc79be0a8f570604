// C ABI of libpagedkv: argument checks, pool geometry, partition choice, kernel launches.
// The declarations and their contracts are in include/pagedkv.h.

#include "pagedkv.h"

#include <math.h>
#include <stdlib.h>

#include <atomic>

#include "pkv_internal.h"

struct pkv_pool {
  char* k;
  char* v;
  size_t layer_bytes;
  int num_layers;
  int num_blocks;
  int num_kv_heads;
  int head_dim;
  int block_size;
  pkv_dtype dtype;
};

namespace {

bool supported_shape(int head_dim, int block_size, pkv_dtype dtype) {
  return (head_dim == 64 || head_dim == 128) && block_size == pkv::kBlock &&
         (dtype == PKV_BF16 || dtype == PKV_FP16);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// a * b with overflow detection (all operands non-negative).
bool mul_ok(size_t a, size_t b, size_t* r) {
  if (a != 0 && b > (size_t)-1 / a) return false;
  *r = a * b;
  return true;
}

// Compute units of the current device (cached); 256 (MI355X) when no device is visible.
int device_cus() {
  static std::atomic<int> cached{0};
  int v = cached.load(std::memory_order_relaxed);
  if (v > 0) return v;
  int dev = 0;
  hipDeviceProp_t prop;
  v = 256;
  if (hipGetDevice(&dev) == hipSuccess && hipGetDeviceProperties(&prop, dev) == hipSuccess &&
      prop.multiProcessorCount > 0) {
    v = prop.multiProcessorCount;
  } else {
    (void)hipGetLastError();
  }
  cached.store(v, std::memory_order_relaxed);
  return v;
}

// Partition size (blocks per decode workgroup, at most kMaxPartBlocks = 256). A workgroup's four
// wavefronts split its partition and combine in LDS; sequences longer than one partition are
// split into near-equal partitions joined by the merge kernel. The longest power-of-two
// partition that still gives every compute unit about two workgroups (eight wavefronts) on the
// longest allowed sequence wins: few long sequences then spread over the whole GPU, while large
// batches keep whole sequences in one workgroup and need no merge at all.
int choose_part_blocks(int num_seqs, int num_q_heads, int num_kv_heads, int max_context_len) {
  const int nb_max = (max_context_len + pkv::kBlock - 1) / pkv::kBlock;
  if (nb_max <= 16) return nb_max > 0 ? nb_max : 1;
  const int group = num_q_heads / num_kv_heads;
  const long tiles = (long)num_seqs * num_kv_heads *
                     ((group + pkv::kMaxGroupTile - 1) / pkv::kMaxGroupTile);
  const long target = 2L * device_cus();
  for (int pb = pkv::kMaxPartBlocks; pb > 16; pb /= 2) {
    if (tiles * ((nb_max + pb - 1) / pb) >= target) return pb < nb_max ? pb : nb_max;
  }
  return 16;
}

int resolve_part_blocks(int num_seqs, int num_q_heads, int num_kv_heads, int max_context_len,
                        int partition_tokens) {
  if (partition_tokens > 0) {
    const int pb = partition_tokens / pkv::kBlock;
    return pb < pkv::kMaxPartBlocks ? pb : pkv::kMaxPartBlocks;
  }
  return choose_part_blocks(num_seqs, num_q_heads, num_kv_heads, max_context_len);
}

bool decode_shape_ok(int num_seqs, int num_q_heads, int num_kv_heads, int max_context_len,
                     int block_size, int partition_tokens) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_context_len < 0) return false;
  if (num_q_heads % num_kv_heads != 0) return false;
  if (block_size <= 0) return false;
  if (partition_tokens < 0 || (partition_tokens > 0 && partition_tokens % block_size != 0))
    return false;
  return true;
}

}  // namespace

extern "C" {

size_t kv_pool_bytes(int num_layers, int num_blocks, int num_kv_heads, int head_dim,
                     int block_size, pkv_dtype dtype) {
  if (num_layers <= 0 || num_blocks <= 0 || num_kv_heads <= 0) return 0;
  if (!supported_shape(head_dim, block_size, dtype)) return 0;
  size_t r = 2;
  const size_t f[5] = {(size_t)num_layers, (size_t)num_blocks, (size_t)num_kv_heads,
                       (size_t)block_size, (size_t)head_dim};
  for (size_t x : f) {
    if (!mul_ok(r, x, &r)) return 0;
  }
  return r;
}

pkv_status kv_pool_create(pkv_pool** out, void* k_base, void* v_base, size_t bytes_each,
                          int num_layers, int num_blocks, int num_kv_heads, int head_dim,
                          int block_size, pkv_dtype dtype) {
  if (out == nullptr) return PKV_ERR_INVALID_ARG;
  *out = nullptr;
  if (k_base == nullptr || v_base == nullptr) return PKV_ERR_INVALID_ARG;
  if (num_layers <= 0 || num_blocks <= 0 || num_kv_heads <= 0) return PKV_ERR_INVALID_ARG;
  if (!supported_shape(head_dim, block_size, dtype)) return PKV_ERR_UNSUPPORTED;
  if (((uintptr_t)k_base & 255u) || ((uintptr_t)v_base & 255u)) return PKV_ERR_ALIGNMENT;
  const size_t need = kv_pool_bytes(num_layers, num_blocks, num_kv_heads, head_dim, block_size,
                                    dtype);
  if (need == 0 || bytes_each < need) return PKV_ERR_INVALID_ARG;
  pkv_pool* p = (pkv_pool*)malloc(sizeof(pkv_pool));
  if (p == nullptr) return PKV_ERR_INVALID_ARG;
  p->k = (char*)k_base;
  p->v = (char*)v_base;
  p->layer_bytes = need / (size_t)num_layers;
  p->num_layers = num_layers;
  p->num_blocks = num_blocks;
  p->num_kv_heads = num_kv_heads;
  p->head_dim = head_dim;
  p->block_size = block_size;
  p->dtype = dtype;
  *out = p;
  return PKV_OK;
}

pkv_status kv_pool_layer(const pkv_pool* pool, int layer, void** k_layer, void** v_layer) {
  if (pool == nullptr || k_layer == nullptr || v_layer == nullptr) return PKV_ERR_INVALID_ARG;
  if (layer < 0 || layer >= pool->num_layers) return PKV_ERR_INVALID_ARG;
  *k_layer = pool->k + (size_t)layer * pool->layer_bytes;
  *v_layer = pool->v + (size_t)layer * pool->layer_bytes;
  return PKV_OK;
}

void kv_pool_destroy(pkv_pool* pool) { free(pool); }

pkv_status reshape_and_cache(const void* key, const void* value, void* k_pool, void* v_pool,
                             const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                             int head_dim, int block_size, int num_blocks, pkv_dtype dtype,
                             hipStream_t stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PKV_ERR_INVALID_ARG;
  if (!supported_shape(head_dim, block_size, dtype)) return PKV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !k_pool || !v_pool || !slot_mapping) return PKV_ERR_INVALID_ARG;
  if (!aligned16(key) || !aligned16(value) || !aligned16(k_pool) || !aligned16(v_pool) ||
      ((uintptr_t)slot_mapping & 7u))
    return PKV_ERR_ALIGNMENT;
  const hipError_t err = pkv::launch_reshape_and_cache(key, value, k_pool, v_pool, slot_mapping,
                                                       num_tokens, num_kv_heads, head_dim, stream);
  return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

int paged_attention_partition_tokens(int num_seqs, int num_q_heads, int num_kv_heads,
                                     int max_context_len, int block_size) {
  if (!decode_shape_ok(num_seqs, num_q_heads, num_kv_heads, max_context_len, block_size, 0) ||
      block_size != pkv::kBlock)
    return 0;
  return choose_part_blocks(num_seqs, num_q_heads, num_kv_heads, max_context_len) * block_size;
}

size_t paged_attention_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                       int head_dim, int block_size, int max_context_len,
                                       int partition_tokens) {
  if (!decode_shape_ok(num_seqs, num_q_heads, num_kv_heads, max_context_len, block_size,
                       partition_tokens) ||
      head_dim <= 0)
    return (size_t)-1;
  if (block_size != pkv::kBlock) return (size_t)-1;
  const int pb = resolve_part_blocks(num_seqs, num_q_heads, num_kv_heads, max_context_len,
                                     partition_tokens);
  const long nb_max = ((long)max_context_len + block_size - 1) / block_size;
  const long max_parts = nb_max > 0 ? (nb_max + pb - 1) / pb : 1;
  if (max_parts <= 1) return 0;
  size_t r = 0;
  if (!mul_ok((size_t)num_seqs * (size_t)num_q_heads, (size_t)max_parts, &r)) return (size_t)-1;
  if (!mul_ok(r, (size_t)(head_dim + 2) * sizeof(float), &r)) return (size_t)-1;
  return r;
}

pkv_status paged_attention_decode(void* out, const void* q, const void* k_pool, const void* v_pool,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  float scale, int num_q_heads, int num_kv_heads, int head_dim,
                                  int block_size, int num_seqs, int max_blocks_per_seq,
                                  int max_context_len, int partition_tokens, pkv_dtype dtype,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!decode_shape_ok(num_seqs, num_q_heads, num_kv_heads, max_context_len, block_size,
                       partition_tokens) ||
      max_blocks_per_seq < 0 || !isfinite(scale))
    return PKV_ERR_INVALID_ARG;
  if (!supported_shape(head_dim, block_size, dtype)) return PKV_ERR_UNSUPPORTED;
  if ((long)max_context_len > (long)max_blocks_per_seq * block_size) return PKV_ERR_INVALID_ARG;
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens)
    return PKV_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) ||
      ((uintptr_t)block_tables & 3u) || ((uintptr_t)context_lens & 3u))
    return PKV_ERR_ALIGNMENT;

  const int pb = resolve_part_blocks(num_seqs, num_q_heads, num_kv_heads, max_context_len,
                                     partition_tokens);
  const long nb_max = ((long)max_context_len + block_size - 1) / block_size;
  const long max_parts = nb_max > 0 ? (nb_max + pb - 1) / pb : 1;
  if (max_parts > 65535) return PKV_ERR_UNSUPPORTED;
  const size_t need = paged_attention_workspace_bytes(num_seqs, num_q_heads, num_kv_heads,
                                                      head_dim, block_size, max_context_len,
                                                      partition_tokens);
  if (need == (size_t)-1) return PKV_ERR_INVALID_ARG;
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return PKV_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return PKV_ERR_ALIGNMENT;

  pkv::DecodeLaunch a;
  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  const size_t o_elems = (size_t)num_seqs * num_q_heads * (size_t)max_parts * head_dim;
  a.ws_o = need > 0 ? (float*)workspace : nullptr;
  a.ws_ml = need > 0 ? (float*)workspace + o_elems : nullptr;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_q_heads / num_kv_heads;
  a.head_tiles = (a.group + pkv::kMaxGroupTile - 1) / pkv::kMaxGroupTile;
  a.max_blocks = max_blocks_per_seq;
  a.part_blocks = pb;
  a.max_parts = (int)max_parts;
  const hipError_t err = pkv::launch_decode(a, head_dim, dtype == PKV_BF16, stream);
  return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

const char* pkv_status_string(pkv_status status) {
  switch (status) {
    case PKV_OK: return "PKV_OK";
    case PKV_ERR_INVALID_ARG: return "PKV_ERR_INVALID_ARG";
    case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED";
    case PKV_ERR_ALIGNMENT: return "PKV_ERR_ALIGNMENT";
    case PKV_ERR_WORKSPACE: return "PKV_ERR_WORKSPACE";
    case PKV_ERR_HIP: return "PKV_ERR_HIP";
  }
  return "PKV_UNKNOWN_STATUS";
}

}  // extern "C"
