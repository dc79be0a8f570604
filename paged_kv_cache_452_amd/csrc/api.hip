// C ABI of libpagedkv: argument checks, pool geometry, grid choice, kernel launches.
// The declarations and their contracts are in include/pagedkv.h.

#include "pagedkv.h"

#include <math.h>
#include <stdlib.h>

#include <atomic>
#include <mutex>

#include "pkv_internal.h"
#include "pkv_link.h"

struct pkv_pool {
  char* base;             // layer 0, block 0, kv head 0: its K tile, then its V tile
  size_t tile_bytes;      // one (block, kv head) tile of K or of V
  size_t layer_bytes;
  int num_layers;
  int num_blocks;
  int num_kv_heads;
  int head_dim;
  int block_size;
  pkv_dtype dtype;
};

namespace {

bool supported_block(int block_size) { return block_size == 16 || block_size == 32; }

bool supported_shape(int head_dim, int block_size, pkv_dtype dtype) {
  return (head_dim == 64 || head_dim == 128) && supported_block(block_size) &&
         (dtype == PKV_BF16 || dtype == PKV_FP16);
}

// Pools may also hold E4M3 codes; q, key, value and out are always 16-bit.
bool supported_pool(int head_dim, int block_size, pkv_dtype dtype) {
  return supported_shape(head_dim, block_size, dtype == PKV_FP8_E4M3 ? PKV_BF16 : dtype);
}

size_t elem_bytes(pkv_dtype dtype) { return dtype == PKV_FP8_E4M3 ? 1 : 2; }

bool valid_scale(float s) { return isfinite(s) && s > 0.f; }

// Device address of a pinned (page-locked, device-mapped) host range [p, p + bytes): both ends
// must be host memory known to the runtime. False for pageable or device memory; a failed query
// is cleared so that it does not surface as the error of a later launch.
bool pinned_device_address(const char* p, size_t bytes, void** dev) {
  const char* ends[2] = {p, p + bytes - 1};
  for (const char* e : ends) {
    hipPointerAttribute_t at;
    if (hipPointerGetAttributes(&at, e) != hipSuccess || at.type != hipMemoryTypeHost) {
      (void)hipGetLastError();
      return false;
    }
  }
  void* d = nullptr;
  if (hipHostGetDevicePointer(&d, (void*)p, 0) != hipSuccess || d == nullptr) {
    (void)hipGetLastError();
    return false;
  }
  *dev = d;
  return true;
}

// Device-visible address of an id array: device memory as is, pinned host memory through its
// device address. False for pageable host memory (a kernel would fault on it) or an unknown
// pointer.
bool device_visible(const int32_t* p, const int32_t** dev) {
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  if (at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeManaged) {
    *dev = p;
    return true;
  }
  if (at.type != hipMemoryTypeHost) return false;
  void* d = nullptr;
  if (hipHostGetDevicePointer(&d, (void*)p, 0) != hipSuccess || d == nullptr) {
    (void)hipGetLastError();
    return false;
  }
  *dev = (const int32_t*)d;
  return true;
}

// True when the host may read p directly: host memory, pinned or pageable (the runtime does not
// know pageable memory, which is fine), or managed memory. False for device memory.
bool host_readable(const void* p) {
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return true;
  }
  return at.type != hipMemoryTypeDevice && at.type != hipMemoryTypeArray;
}

// Range weight of decode workgroups on odd-numbered XCDs (even ones weigh pkv::kEvenWeight): the
// default below, or PKV_ODD_XCD_WEIGHT from the environment, clamped to
// [kEvenWeight / 2, kEvenWeight]. Read once, at the first decode call of the process: the weight
// moves the range boundaries and with them the rounding order of split streams, so every call of
// one process must use the same value for its results to be reproducible.
constexpr int kDefaultOddXcdWeight = 900;
int odd_xcd_weight() {
  static const int weight = [] {
    int v = kDefaultOddXcdWeight;
    if (const char* e = getenv("PKV_ODD_XCD_WEIGHT")) v = atoi(e);
    return v < pkv::kEvenWeight / 2 ? pkv::kEvenWeight / 2
                                    : v > pkv::kEvenWeight ? pkv::kEvenWeight : v;
  }();
  return weight;
}

// Bytes of one block's region in one layer: the K and V tiles of all its kv heads.
size_t block_bytes_of(const pkv_pool* p) {
  return (size_t)p->num_kv_heads * 2 * p->tile_bytes;
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

// Workgroups of a decode launch when the caller leaves the choice to the library: enough to
// fill every compute unit (kWorkgroupsPerCU resident each), but no more than one per 64 block
// positions of the largest possible batch (16 per wavefront), so that small batches are not cut
// into slivers. The kernel spreads the actual positions evenly over the wavefronts it is given.
int default_workgroups(int num_seqs, int num_q_heads, int num_kv_heads, int max_context_len) {
  const int group = num_q_heads / num_kv_heads;
  const long streams = (long)num_seqs * num_kv_heads *
                       ((group + pkv::kMaxGroupTile - 1) / pkv::kMaxGroupTile);
  const long nb_max = ((long)max_context_len + pkv::kBlock - 1) / pkv::kBlock;
  const long positions = streams * nb_max;
  const long full = (long)pkv::kWorkgroupsPerCU * device_cus();
  long g = (positions + 63) / 64;  // >= 16 blocks per wavefront
  // Few, short streams: at least one workgroup per stream, so that they run side by side instead
  // of one after another inside a workgroup (on the tiny 4-sequence batch: 10 us instead of 28).
  if (g < streams) g = streams;
  if (g > full) g = full;
  return g > 0 ? (int)g : 1;
}

constexpr int kMaxWorkgroups = 1 << 20;

bool decode_shape_ok(int num_seqs, int num_q_heads, int num_kv_heads, int max_context_len,
                     int block_size, int num_workgroups) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_context_len < 0) return false;
  if (num_q_heads % num_kv_heads != 0) return false;
  if (block_size <= 0) return false;
  if (num_workgroups < 0 || num_workgroups > kMaxWorkgroups) return false;
  return true;
}

int resolve_workgroups(int num_seqs, int num_q_heads, int num_kv_heads, int max_context_len,
                       int num_workgroups) {
  return num_workgroups > 0
             ? num_workgroups
             : default_workgroups(num_seqs, num_q_heads, num_kv_heads, max_context_len);
}

// Workspace for `grid` workgroups (one range each): (m, l) and partial outputs from the start,
// arrival counters in the last 4 bytes per workgroup of the caller's buffer. Keeping the
// counters at the end means calls with fewer workgroups never write partials over the counters of
// calls with more, so one zero-filled buffer serves any sequence of calls it is large enough for.
size_t counter_bytes(int grid) { return ((size_t)grid * sizeof(unsigned) + 255) & ~(size_t)255; }
size_t ml_bytes(int grid) { return (size_t)grid * 2 * pkv::kMaxGroupTile * 2 * sizeof(float); }
size_t workspace_bytes_for(int grid, int head_dim) {
  return counter_bytes(grid) + ml_bytes(grid) +
         (size_t)grid * 2 * pkv::kMaxGroupTile * head_dim * sizeof(float);
}

}  // namespace

extern "C" {

size_t kv_pool_bytes(int num_layers, int num_blocks, int num_kv_heads, int head_dim,
                     int block_size, pkv_dtype dtype) {
  if (num_layers <= 0 || num_blocks <= 0 || num_kv_heads <= 0) return 0;
  if (!supported_pool(head_dim, block_size, dtype)) return 0;
  size_t r = 2 * elem_bytes(dtype);  // K and V
  const size_t f[5] = {(size_t)num_layers, (size_t)num_blocks, (size_t)num_kv_heads,
                       (size_t)block_size, (size_t)head_dim};
  for (size_t x : f) {
    if (!mul_ok(r, x, &r)) return 0;
  }
  return r;
}

pkv_status kv_pool_create(pkv_pool** out, void* base, size_t bytes, int num_layers,
                          int num_blocks, int num_kv_heads, int head_dim, int block_size,
                          pkv_dtype dtype) {
  if (out == nullptr) return PKV_ERR_INVALID_ARG;
  *out = nullptr;
  if (base == nullptr) return PKV_ERR_INVALID_ARG;
  if (num_layers <= 0 || num_blocks <= 0 || num_kv_heads <= 0) return PKV_ERR_INVALID_ARG;
  if (!supported_pool(head_dim, block_size, dtype)) return PKV_ERR_UNSUPPORTED;
  if ((uintptr_t)base & 255u) return PKV_ERR_ALIGNMENT;
  const size_t need = kv_pool_bytes(num_layers, num_blocks, num_kv_heads, head_dim, block_size,
                                    dtype);
  if (need == 0 || bytes < need) return PKV_ERR_INVALID_ARG;
  pkv_pool* p = (pkv_pool*)malloc(sizeof(pkv_pool));
  if (p == nullptr) return PKV_ERR_INVALID_ARG;
  p->base = (char*)base;
  p->tile_bytes = (size_t)block_size * head_dim * elem_bytes(dtype);
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
  char* k = pool->base + (size_t)layer * pool->layer_bytes;
  *k_layer = k;
  *v_layer = k + pool->tile_bytes;
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
                                                       num_tokens, num_kv_heads, head_dim,
                                                       block_size, num_blocks, stream);
  return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

pkv_status reshape_and_cache_fp8(const void* key, const void* value, void* k_pool, void* v_pool,
                                 const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                                 int head_dim, int block_size, int num_blocks, pkv_dtype src_dtype,
                                 float k_scale, float v_scale, hipStream_t stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PKV_ERR_INVALID_ARG;
  if (!valid_scale(k_scale) || !valid_scale(v_scale)) return PKV_ERR_INVALID_ARG;
  if (!supported_shape(head_dim, block_size, src_dtype)) return PKV_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !k_pool || !v_pool || !slot_mapping) return PKV_ERR_INVALID_ARG;
  if (!aligned16(key) || !aligned16(value) || !aligned16(k_pool) || !aligned16(v_pool) ||
      ((uintptr_t)slot_mapping & 7u))
    return PKV_ERR_ALIGNMENT;
  const float one = 1.0f;
  const hipError_t err = pkv::launch_reshape_and_cache_fp8(
      key, value, k_pool, v_pool, slot_mapping, num_tokens, num_kv_heads, head_dim, block_size,
      num_blocks, src_dtype == PKV_BF16, one / k_scale, one / v_scale, stream);
  return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

pkv_status copy_blocks(const pkv_pool* pool, const int32_t* src_blocks, const int32_t* dst_blocks,
                       int num_copies, hipStream_t stream) {
  if (pool == nullptr || num_copies < 0 || num_copies > 65535) return PKV_ERR_INVALID_ARG;
  if (num_copies == 0) return PKV_OK;
  if (src_blocks == nullptr || dst_blocks == nullptr) return PKV_ERR_INVALID_ARG;
  if (((uintptr_t)src_blocks & 3u) || ((uintptr_t)dst_blocks & 3u)) return PKV_ERR_ALIGNMENT;
  if (pool->num_layers > 32767) return PKV_ERR_UNSUPPORTED;
  const int32_t* src_dev = nullptr;
  const int32_t* dst_dev = nullptr;
  if (!device_visible(src_blocks, &src_dev) || !device_visible(dst_blocks, &dst_dev))
    return PKV_ERR_INVALID_ARG;
  pkv::BlockCopy c;
  c.src = pool->base;
  c.dst = pool->base;
  c.src_layer_bytes = c.dst_layer_bytes = pool->layer_bytes;
  c.block_bytes = block_bytes_of(pool);
  c.src_ids = src_dev;
  c.dst_ids = dst_dev;
  c.src_blocks = c.dst_blocks = pool->num_blocks;
  const hipError_t err = pkv::launch_block_copy(c, pool->num_layers, num_copies, stream);
  return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

pkv_status swap_blocks(const pkv_pool* device_pool, const pkv_pool* host_pool,
                       const int32_t* src_blocks, const int32_t* dst_blocks, int num_pairs,
                       pkv_swap_dir direction, hipStream_t stream) {
  if (device_pool == nullptr || host_pool == nullptr || num_pairs < 0 || num_pairs > 65535)
    return PKV_ERR_INVALID_ARG;
  if (direction != PKV_SWAP_OUT && direction != PKV_SWAP_IN) return PKV_ERR_INVALID_ARG;
  const pkv_pool& d = *device_pool;
  const pkv_pool& h = *host_pool;
  if (d.num_layers != h.num_layers || d.num_kv_heads != h.num_kv_heads ||
      d.head_dim != h.head_dim || d.block_size != h.block_size || d.dtype != h.dtype)
    return PKV_ERR_INVALID_ARG;
  if (num_pairs == 0) return PKV_OK;
  if (src_blocks == nullptr || dst_blocks == nullptr) return PKV_ERR_INVALID_ARG;
  if (((uintptr_t)src_blocks & 3u) || ((uintptr_t)dst_blocks & 3u)) return PKV_ERR_ALIGNMENT;
  if (d.num_layers > 32767) return PKV_ERR_UNSUPPORTED;
  // The host pool must be pinned, device-mapped memory: refuse anything else instead of letting
  // the kernel fault on it, and use the device addresses of its bases.
  const size_t host_bytes = h.layer_bytes * (size_t)h.num_layers;
  void* hbase = nullptr;
  if (!pinned_device_address(h.base, host_bytes, &hbase)) return PKV_ERR_INVALID_ARG;
  const int32_t* src_dev = nullptr;
  const int32_t* dst_dev = nullptr;
  if (!device_visible(src_blocks, &src_dev) || !device_visible(dst_blocks, &dst_dev))
    return PKV_ERR_INVALID_ARG;
  pkv::BlockCopy c;
  const bool out = direction == PKV_SWAP_OUT;
  c.src = out ? d.base : (const char*)hbase;
  c.dst = out ? (char*)hbase : d.base;
  c.src_layer_bytes = out ? d.layer_bytes : h.layer_bytes;
  c.dst_layer_bytes = out ? h.layer_bytes : d.layer_bytes;
  c.block_bytes = block_bytes_of(&d);
  c.src_ids = src_dev;
  c.dst_ids = dst_dev;
  c.src_blocks = out ? d.num_blocks : h.num_blocks;
  c.dst_blocks = out ? h.num_blocks : d.num_blocks;
  const hipError_t err = pkv::launch_block_copy_link(c, d.num_layers, num_pairs, stream);
  return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

pkv_status swap_blocks_dma(const pkv_pool* device_pool, const pkv_pool* host_pool,
                           const int32_t* src_blocks, const int32_t* dst_blocks, int num_pairs,
                           pkv_swap_dir direction, hipStream_t stream) {
  if (device_pool == nullptr || host_pool == nullptr || num_pairs < 0 || num_pairs > 65535)
    return PKV_ERR_INVALID_ARG;
  if (direction != PKV_SWAP_OUT && direction != PKV_SWAP_IN) return PKV_ERR_INVALID_ARG;
  const pkv_pool& d = *device_pool;
  const pkv_pool& h = *host_pool;
  if (d.num_layers != h.num_layers || d.num_kv_heads != h.num_kv_heads ||
      d.head_dim != h.head_dim || d.block_size != h.block_size || d.dtype != h.dtype)
    return PKV_ERR_INVALID_ARG;
  if (num_pairs == 0) return PKV_OK;
  if (src_blocks == nullptr || dst_blocks == nullptr) return PKV_ERR_INVALID_ARG;
  if (!host_readable(src_blocks) || !host_readable(dst_blocks)) return PKV_ERR_INVALID_ARG;
  // The copy engines take the pinned host pool by its host address; pageable memory is refused.
  void* hdev = nullptr;
  if (!pinned_device_address(h.base, h.layer_bytes * (size_t)h.num_layers, &hdev))
    return PKV_ERR_INVALID_ARG;
  const bool out = direction == PKV_SWAP_OUT;
  const int src_n = out ? d.num_blocks : h.num_blocks;
  const int dst_n = out ? h.num_blocks : d.num_blocks;
  // Every id is checked before anything is enqueued: a refused call moves nothing.
  for (int i = 0; i < num_pairs; ++i) {
    if (src_blocks[i] < 0 || src_blocks[i] >= src_n || dst_blocks[i] < 0 ||
        dst_blocks[i] >= dst_n)
      return PKV_ERR_INVALID_ARG;
  }
  const size_t block_bytes = block_bytes_of(&d);
  const char* src_base = out ? d.base : h.base;
  char* dst_base = out ? h.base : d.base;
  const size_t src_pitch = out ? d.layer_bytes : h.layer_bytes;
  const size_t dst_pitch = out ? h.layer_bytes : d.layer_bytes;
  const hipMemcpyKind kind = out ? hipMemcpyDeviceToHost : hipMemcpyHostToDevice;
  // One strided copy per block: its region in every layer (block_bytes wide, num_layers rows, one
  // layer stride apart on each side).
  for (int i = 0; i < num_pairs; ++i) {
    const char* src = src_base + (size_t)src_blocks[i] * block_bytes;
    char* dst = dst_base + (size_t)dst_blocks[i] * block_bytes;
    if (hipMemcpy2DAsync(dst, dst_pitch, src, src_pitch, block_bytes, (size_t)d.num_layers, kind,
                         stream) != hipSuccess)
      return PKV_ERR_HIP;
  }
  return PKV_OK;
}

int paged_attention_num_workgroups(int num_seqs, int num_q_heads, int num_kv_heads,
                                   int max_context_len, int block_size) {
  if (!decode_shape_ok(num_seqs, num_q_heads, num_kv_heads, max_context_len, block_size, 0) ||
      !supported_block(block_size))
    return 0;
  return default_workgroups(num_seqs, num_q_heads, num_kv_heads, max_context_len);
}

size_t paged_attention_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                       int head_dim, int block_size, int max_context_len,
                                       int num_workgroups) {
  if (!decode_shape_ok(num_seqs, num_q_heads, num_kv_heads, max_context_len, block_size,
                       num_workgroups) ||
      head_dim <= 0 || !supported_block(block_size))
    return (size_t)-1;
  const int grid = resolve_workgroups(num_seqs, num_q_heads, num_kv_heads, max_context_len,
                                      num_workgroups);
  return workspace_bytes_for(grid, head_dim);
}

}  // extern "C"

// ---- Library-owned decode scratch for callers that cannot allocate ----
// One statically sized device array per GPU the library runs on (each device holds its own copy
// at its own address until the process ends). It takes the place of the caller's workspace:
// split-stream partials from its start, arrival counters in its last 4 bytes per workgroup. In
// host code `scratch` is only a stand-in for the symbol; its device address on the current device
// comes from hipGetSymbolAddress and is the only form passed to kernels.
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

static_assert(PKV_NOALLOC_SCRATCH_BYTES % 256 == 0, "the scratch size is a whole number of lines");

namespace {

// Decode, plain or fused with the append of each sequence's newest token (new_k / new_v non-null:
// rows [num_seqs][num_kv_heads][head_dim] of q's element type).
pkv_status decode_impl(void* out, const void* q, const void* new_k, const void* new_v,
                       const void* k_pool, const void* v_pool,
                       const int32_t* block_tables, const int32_t* context_lens, float scale,
                       bool kv_fp8, float k_scale, float v_scale, int num_q_heads,
                       int num_kv_heads, int head_dim, int block_size, int num_seqs,
                       int max_blocks_per_seq, int max_context_len, int num_workgroups,
                       pkv_dtype dtype, void* workspace, size_t workspace_bytes,
                       hipStream_t stream) {
  if (!decode_shape_ok(num_seqs, num_q_heads, num_kv_heads, max_context_len, block_size,
                       num_workgroups) ||
      max_blocks_per_seq < 0 || !isfinite(scale) || !valid_scale(k_scale) ||
      !valid_scale(v_scale))
    return PKV_ERR_INVALID_ARG;
  if (!supported_shape(head_dim, block_size, dtype)) return PKV_ERR_UNSUPPORTED;
  if ((long)max_context_len > (long)max_blocks_per_seq * block_size) return PKV_ERR_INVALID_ARG;
  if (num_seqs == 0) return PKV_OK;
  if (num_seqs > pkv::kMaxSeqs) return PKV_ERR_UNSUPPORTED;
  const int group = num_q_heads / num_kv_heads;
  const int head_tiles = (group + pkv::kMaxGroupTile - 1) / pkv::kMaxGroupTile;
  // Flattened block positions and token counts are 32-bit on the device.
  if (max_blocks_per_seq > 2147483647 / block_size) return PKV_ERR_UNSUPPORTED;
  if ((long double)num_seqs * max_blocks_per_seq * (block_size / pkv::kBlock) * num_kv_heads *
          head_tiles >= 2147483647.0L)
    return PKV_ERR_UNSUPPORTED;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens)
    return PKV_ERR_INVALID_ARG;
  const bool append = new_k != nullptr || new_v != nullptr;
  if (append && (new_k == nullptr || new_v == nullptr)) return PKV_ERR_INVALID_ARG;
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) ||
      ((uintptr_t)block_tables & 3u) || ((uintptr_t)context_lens & 3u) ||
      (append && (!aligned16(new_k) || !aligned16(new_v))))
    return PKV_ERR_ALIGNMENT;

  const int grid = resolve_workgroups(num_seqs, num_q_heads, num_kv_heads, max_context_len,
                                      num_workgroups);
  const size_t need = workspace_bytes_for(grid, head_dim);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return PKV_ERR_WORKSPACE;
  if (need > 0 && ((uintptr_t)workspace & 255u)) return PKV_ERR_ALIGNMENT;

  pkv::DecodeLaunch a;
  a.out = out;
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  char* ws = (char*)workspace;
  a.ws_ml = need > 0 ? (float*)ws : nullptr;
  a.ws_o = need > 0 ? (float*)(ws + ml_bytes(grid)) : nullptr;
  a.counters = need > 0 ? (unsigned*)(ws + (workspace_bytes & ~(size_t)3) -
                                      (size_t)grid * sizeof(unsigned))
                        : nullptr;
  a.scale_log2 = scale * k_scale * 1.4426950408889634f;
  a.v_scale = v_scale;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.head_tiles = head_tiles;
  a.max_blocks = max_blocks_per_seq;
  a.max_tokens = max_blocks_per_seq * block_size;
  a.sub_shift = block_size == 32 ? 1 : 0;
  a.new_k = new_k;
  a.new_v = new_v;
  a.odd_weight = odd_xcd_weight();
  a.may_halve = num_workgroups == 0 && grid == pkv::kWorkgroupsPerCU * device_cus() &&
                (long)num_seqs * num_kv_heads * head_tiles <= grid;
  const float one = 1.0f;
  a.k_inv = one / k_scale;
  a.v_inv = one / v_scale;
  const hipError_t err =
      pkv::launch_decode(a, grid, head_dim, dtype == PKV_BF16, kv_fp8, append, stream);
  return err == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

constexpr int kMaxDevices = 64;
constexpr int kScratchCounterWords = 4096;  // counters cleared at set-up: more than any grid uses

__global__ void clear_words_kernel(unsigned* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Device address of the scratch array on the current device. The first call on a device looks it
// up and clears the counter words with a fill kernel on `stream` (a kernel, so that the clear is
// also valid inside a stream being captured into a graph); later calls rely on every completed
// decode leaving its counters zero.
pkv_status scratch_address(hipStream_t stream, void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return PKV_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return PKV_ERR_HIP;
    }
    unsigned* counters = (unsigned*)((char*)p + PKV_NOALLOC_SCRATCH_BYTES) - kScratchCounterWords;
    hipLaunchKernelGGL(clear_words_kernel, dim3((kScratchCounterWords + 255) / 256), dim3(256), 0,
                       stream, counters, kScratchCounterWords);
    if (hipGetLastError() != hipSuccess) return PKV_ERR_HIP;
    addr[dev] = p;
  }
  *out = addr[dev];
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status paged_attention_decode_noalloc(void* out, const void* q, const void* k_pool,
                                          const void* v_pool, const int32_t* block_tables,
                                          const int32_t* context_lens, float scale,
                                          int num_q_heads, int num_kv_heads, int head_dim,
                                          int block_size, int num_seqs, int max_blocks_per_seq,
                                          int max_context_len, int num_workgroups,
                                          pkv_dtype dtype, hipStream_t stream) {
  if (!decode_shape_ok(num_seqs, num_q_heads, num_kv_heads, max_context_len, block_size,
                       num_workgroups))
    return PKV_ERR_INVALID_ARG;
  if (!supported_shape(head_dim, block_size, dtype)) return PKV_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PKV_OK;
  const int grid = resolve_workgroups(num_seqs, num_q_heads, num_kv_heads, max_context_len,
                                      num_workgroups);
  if (workspace_bytes_for(grid, head_dim) > PKV_NOALLOC_SCRATCH_BYTES ||
      grid > kScratchCounterWords)
    return PKV_ERR_WORKSPACE;
  void* ws = nullptr;
  const pkv_status st = scratch_address(stream, &ws);
  if (st != PKV_OK) return st;
  return decode_impl(out, q, nullptr, nullptr, k_pool, v_pool, block_tables, context_lens, scale,
                     false, 1.0f, 1.0f, num_q_heads, num_kv_heads, head_dim, block_size, num_seqs,
                     max_blocks_per_seq, max_context_len, num_workgroups, dtype, ws,
                     PKV_NOALLOC_SCRATCH_BYTES, stream);
}

pkv_status paged_attention_decode(void* out, const void* q, const void* k_pool, const void* v_pool,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  float scale, int num_q_heads, int num_kv_heads, int head_dim,
                                  int block_size, int num_seqs, int max_blocks_per_seq,
                                  int max_context_len, int num_workgroups, pkv_dtype dtype,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_impl(out, q, nullptr, nullptr, k_pool, v_pool, block_tables, context_lens, scale,
                     false, 1.0f, 1.0f, num_q_heads, num_kv_heads, head_dim, block_size, num_seqs,
                     max_blocks_per_seq, max_context_len, num_workgroups, dtype, workspace,
                     workspace_bytes, stream);
}

pkv_status paged_attention_decode_append(void* out, const void* q, const void* key,
                                         const void* value, void* k_pool, void* v_pool,
                                         const int32_t* block_tables, const int32_t* context_lens,
                                         float scale, int num_q_heads, int num_kv_heads,
                                         int head_dim, int block_size, int num_seqs,
                                         int max_blocks_per_seq, int max_context_len,
                                         int num_workgroups, pkv_dtype dtype, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
  if (num_seqs > 0 && (key == nullptr || value == nullptr)) return PKV_ERR_INVALID_ARG;
  return decode_impl(out, q, key, value, k_pool, v_pool, block_tables, context_lens, scale, false,
                     1.0f, 1.0f, num_q_heads, num_kv_heads, head_dim, block_size, num_seqs,
                     max_blocks_per_seq, max_context_len, num_workgroups, dtype, workspace,
                     workspace_bytes, stream);
}

pkv_status paged_attention_decode_append_fp8(void* out, const void* q, const void* key,
                                             const void* value, void* k_pool, void* v_pool,
                                             const int32_t* block_tables,
                                             const int32_t* context_lens, float scale,
                                             float k_scale, float v_scale, int num_q_heads,
                                             int num_kv_heads, int head_dim, int block_size,
                                             int num_seqs, int max_blocks_per_seq,
                                             int max_context_len, int num_workgroups,
                                             pkv_dtype dtype, void* workspace,
                                             size_t workspace_bytes, hipStream_t stream) {
  if (num_seqs > 0 && (key == nullptr || value == nullptr)) return PKV_ERR_INVALID_ARG;
  return decode_impl(out, q, key, value, k_pool, v_pool, block_tables, context_lens, scale, true,
                     k_scale, v_scale, num_q_heads, num_kv_heads, head_dim, block_size, num_seqs,
                     max_blocks_per_seq, max_context_len, num_workgroups, dtype, workspace,
                     workspace_bytes, stream);
}

pkv_status paged_attention_decode_fp8(void* out, const void* q, const void* k_pool,
                                      const void* v_pool, const int32_t* block_tables,
                                      const int32_t* context_lens, float scale, float k_scale,
                                      float v_scale, int num_q_heads, int num_kv_heads,
                                      int head_dim, int block_size, int num_seqs,
                                      int max_blocks_per_seq, int max_context_len,
                                      int num_workgroups, pkv_dtype dtype, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  return decode_impl(out, q, nullptr, nullptr, k_pool, v_pool, block_tables, context_lens, scale,
                     true, k_scale, v_scale, num_q_heads, num_kv_heads, head_dim, block_size, num_seqs,
                     max_blocks_per_seq, max_context_len, num_workgroups, dtype, workspace,
                     workspace_bytes, stream);
}

const char* pkv_status_string(pkv_status status) {
  switch (status) {
    case PKV_OK: return "PKV_OK";
    case PKV_ERR_INVALID_ARG: return "PKV_ERR_INVALID_ARG";
    case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED";
    case PKV_ERR_ALIGNMENT: return "PKV_ERR_ALIGNMENT";
    case PKV_ERR_WORKSPACE: return "PKV_ERR_WORKSPACE";
    case PKV_ERR_HIP: return "PKV_ERR_HIP";
    case PKV_ERR_NO_BLOCKS: return "PKV_ERR_NO_BLOCKS";
  }
  return "PKV_UNKNOWN_STATUS";
}

}  // extern "C"
