/*
 * pagedkv.h — C ABI of libpagedkv: PagedAttention decode on AMD Instinct MI355X (gfx950).
 *
 * The library implements the decode step of paged attention. A sequence's keys and values live in
 * fixed-size blocks of `block_size` tokens, scattered over one shared physical block pool; row s
 * of the block tables holds, at entry j, the physical block id of tokens j*B .. j*B+B-1.
 * The attention kernel takes the block table as an argument and gathers K and V through it in
 * place, with no staging copy into contiguous memory.
 *   - "KV-Cache Management and PagedAttention" (adversariallm.ai), section
 *     "PagedAttention: treat the cache like virtual memory" (block table, block size 16,
 *     the tok 0..40 -> phys [7,3,9] diagram).
 *   - "PagedAttention and KV Cache Management" (blog.sejan.dev), sections
 *     "PagedAttention: OS Virtual Memory Architecture for GPUs" (physical pool, block table),
 *     "How Block Paging Operates During Generation" (boundary allocation; block byte size spans
 *     all layers) and "Under the Hood: The PagedAttention CUDA Kernel"
 *     (the kernel resolves each logical block through the table, then takes the softmax over the
 *     keys it gathered).
 *
 * Conventions for every entry point
 *   - Device pointers are HIP device addresses owned by the caller. The library never allocates
 *     or frees device memory. A `pkv_pool` object holds host-side geometry only.
 *   - Calls that take a `stream` enqueue their kernels on it and return without synchronising.
 *     A NULL stream is the HIP null stream.
 *   - Argument errors found on the host come back as a negative `pkv_status` and nothing is
 *     launched. A failed kernel launch returns PKV_ERR_HIP. Nothing is thrown across the ABI.
 *   - Device-resident indices (block table entries, slots) are NOT validated: the block ids a
 *     sequence uses (the first ceil(n / block_size) of its row) must lie in [0, num_blocks), and
 *     slots must be distinct within one call. Violations are undefined behaviour (out-of-bounds
 *     device accesses). Context lengths are clamped to [0, max_blocks_per_seq*block_size] (a
 *     negative length decodes as an empty sequence), but the clamped length must still name valid
 *     blocks. max_context_len sizes the grid and workspace; lengths above it decode correctly.
 *     On request, paged_attention_check_inputs counts violations on the device (a debug aid).
 *   - A call's output (out; the pool for the scatter calls) must not overlap its other inputs:
 *     the kernels read inputs while they write the output.
 *   - Stateless and thread-safe: concurrent calls are fine as long as their outputs do not alias.
 *
 * Element types: bf16 (PKV_BF16) or IEEE fp16 (PKV_FP16); q, key, value, the pools and out all use
 * the same type. Accumulation is fp32. The softmax weights enter the weighted sum of V as a bf16
 * value plus a bf16 residual for bf16 pools (fp32-level precision), and as one fp16 value for fp16
 * pools (relative error at most 2^-12).
 *
 * Supported shapes: head_dim in {64, 128}; block_size in {16, 32} ("PagedAttention and KV Cache
 * Management", section "PagedAttention: OS Virtual Memory Architecture for GPUs": B = 16 or 32);
 * num_q_heads % num_kv_heads == 0
 * (query head h reads kv head h / (num_q_heads / num_kv_heads): consecutive query heads form one
 * group); any group size.
 *
 * ---------------------------------------------------------------------------------------------
 * KV pool layout (the one data format this ABI defines)
 *
 * One pool holds K and V of every layer: [layer][block][kv_head][K tile, V tile], one tile = B*D
 * elements (4 KiB for D=128, B=16 in 16-bit). Key element (layer L, block b, kv head h, token
 * slot t in [0,B), dim d in [0,D)) lives at element index
 *
 *     ((L * num_blocks + b) * num_kv_heads + h) * (2 * B * D) + tile_offset_K(t, d)
 *
 * and the value element at the same index plus B * D, with tile_offset_V. So the K and V tiles of
 * one (block, kv head) are one contiguous region of 2 * B * D elements (8 KiB for D=128, B=16),
 * and a block's region in one layer (all kv heads) is contiguous too. Tile bases are 4 KiB
 * aligned when the pool base is. The kernels take one layer's K and V *planes*: k_pool points at
 * the K tile of (block 0, head 0) of that layer and v_pool at its V tile (kv_pool_layer gives
 * both; v_pool = k_pool + B * D elements), and in each plane the tile of (b, h) starts
 * 2 * (b * num_kv_heads + h) tiles from the plane's base.
 * Inside a tile, the B tokens are split
 * into sub-tiles of 16 tokens (sub = t / 16, u = t % 16), each 16*D elements; within a sub-tile:
 *
 *   K tile:  k_off(u, d) = (d / 8) * 128 + u * 8 + (d % 8)
 *            -> [D/8][16 tokens][8 dims]: eight consecutive dims of one token are one 16-byte
 *               chunk, and the 16 tokens' chunks for the same eight dims are contiguous.
 *   V tile:  v_off(u, d) = ((((d / 32) * 4 + u / 4) * 16 + d % 16) * 2 + (d / 16) % 2) * 4 + u % 4
 *            -> [D/32][4 token quads][16 dims][2 dim halves][4 tokens]: four consecutive tokens of
 *               one dim are one 8-byte chunk.
 *   tile_offset_K(t, d) = (t / 16) * 16 * D + k_off(t % 16, d)   (tile_offset_V: v_off)
 *
 * Worked examples (D = 128, B = 16): K (t=1,d=0) -> 8; K (t=0,d=8) -> 128; K (t=5,d=37) -> 557;
 * V (t=1,d=0) -> 1; V (t=0,d=1) -> 8; V (t=0,d=16) -> 4; V (t=5,d=37) -> 681;
 * V (t=15,d=127) -> 2047.
 * With these layouts one wavefront reads a whole K or V tile as 64 lanes x 16 bytes per load
 * instruction, every instruction covering one contiguous, 1 KiB aligned range, and each lane's
 * 16 bytes are already the operand of one gfx950 matrix-core instruction.
 *
 * A slot is `physical_block * block_size + t` (token slot t of that block).
 *
 * fp8 pools (PKV_FP8_E4M3) use the same [layer][block][kv_head][K tile, V tile] order and
 * 16-token sub-tiles, one byte per element, with these orders inside a sub-tile (byte offsets):
 *   K8 tile: k8_off(u, d) = (d / 64) * 1024 + (16 * ((d / 8) % 4) + u) * 16 + ((d / 32) % 2) * 8
 *                           + d % 8
 *   V8 tile: v8_off(u, d) = (d / 64) * 1024 + ((u / 4) * 16 + d % 16) * 16 + ((d / 16) % 4) * 4
 *                           + u % 4
 * Worked examples (D = 128, B = 16): K8 (t=1,d=0) -> 16; K8 (t=0,d=8) -> 256; K8 (t=0,d=32) -> 8;
 * K8 (t=5,d=37) -> 93; V8 (t=0,d=1) -> 16; V8 (t=0,d=16) -> 4; V8 (t=5,d=37) -> 345.
 * Each lane's 16 bytes are again one contiguous piece of a 1 KiB load that expands, code by
 * code, into its matrix-core operands.
 * ---------------------------------------------------------------------------------------------
 */
#ifndef PAGEDKV_H_
#define PAGEDKV_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1, /* null pointer, negative size, bad head ratio, out-of-range layer */
  PKV_ERR_UNSUPPORTED = -2, /* head_dim / block_size / dtype this build has no kernel for */
  PKV_ERR_ALIGNMENT = -3,   /* a device pointer not 16-byte aligned */
  PKV_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than paged_attention_workspace_bytes */
  PKV_ERR_HIP = -5,         /* the HIP runtime reported an error at launch */
  PKV_ERR_NO_BLOCKS = -6    /* the block manager's free list cannot supply the blocks needed */
} pkv_status;

/* Element types. q, key, value and out are bf16 or fp16. Pools are bf16 or fp16 (the same type as
 * q), or E4M3 codes (PKV_FP8_E4M3, see reshape_and_cache_fp8 / paged_attention_decode_fp8). */
typedef enum { PKV_BF16 = 0, PKV_FP16 = 1, PKV_FP8_E4M3 = 2 } pkv_dtype;

/* Opaque host-side description of one KV pool holding K and V of every layer. */
typedef struct pkv_pool pkv_pool;

/*
 * Bytes of the pool (K and V of all layers):
 *   2 * num_layers * num_blocks * num_kv_heads * block_size * head_dim * element bytes
 * (2 for bf16/fp16, 1 for PKV_FP8_E4M3).
 * This is the per-token KV size of the sizing formula ("KV-Cache Management and PagedAttention",
 * section "Why the cache exists, and why it's so hungry"; "PagedAttention and KV Cache
 * Management", section "The KV Cache Size Equation") times block_size * num_blocks tokens.
 * Returns 0 for any non-positive argument, an unsupported shape, or on size_t overflow.
 */
size_t kv_pool_bytes(int num_layers, int num_blocks, int num_kv_heads, int head_dim, int block_size,
                     pkv_dtype dtype);

/*
 * Describe a caller-allocated pool (`bytes` bytes at `base`, laid out as above): the one shared
 * pool of fixed-size physical blocks that every sequence's table points into ("PagedAttention and
 * KV Cache Management", section "PagedAttention: OS Virtual Memory Architecture for GPUs": the
 * cache is carved into equal blocks in one physical pool; "KV-Cache Management and
 * PagedAttention", section "PagedAttention: treat the cache like virtual memory": any free block
 * can hold any sequence's tokens). One block id names the same slot range in every layer, as
 * the block byte size in "How Block Paging Operates During Generation" (item 3) spans all layers.
 * Checks: non-NULL, 256-byte aligned base, bytes >= kv_pool_bytes(...), supported shape. On
 * success *out receives a new host object (free it with kv_pool_destroy). The memory stays owned
 * by the caller and must outlive the object. No device work is done.
 * Errors: PKV_ERR_INVALID_ARG (NULL out or base, non-positive size, bytes too small, host
 * allocation failure), PKV_ERR_UNSUPPORTED (head_dim, block_size or dtype), PKV_ERR_ALIGNMENT.
 */
pkv_status kv_pool_create(pkv_pool** out, void* base, size_t bytes, int num_layers,
                          int num_blocks, int num_kv_heads, int head_dim, int block_size,
                          pkv_dtype dtype);

/* Addresses of layer `layer`'s K and V planes: k_layer = base + layer * (kv_pool_bytes / layers),
 * v_layer = k_layer + one tile (block_size * head_dim elements). Each layer keeps its own keys and
 * values for the same block ids ("KV-Cache Management and PagedAttention", section "Why the cache
 * exists, and why it's so hungry": one key and one value vector per token, head and layer).
 * The decode and scatter calls take these two addresses. PKV_ERR_INVALID_ARG for a NULL argument
 * or a layer outside [0, num_layers); nothing is written then. */
pkv_status kv_pool_layer(const pkv_pool* pool, int layer, void** k_layer, void** v_layer);

/* Frees the host object (NULL is a no-op). Does not touch device memory. */
void kv_pool_destroy(pkv_pool* pool);

/*
 * Scatter one step's new keys and values into the pool: for every token i in [0, num_tokens)
 * with slot = slot_mapping[i] >= 0, and every kv head h,
 *     K_pool[slot / block_size][h][slot % block_size][:] = key[i][h][:]   (same for V),
 * bit-exact. Tokens with a negative slot are skipped. This is the device half of boundary
 * allocation: the host block manager chooses the slot (the current block, or a block popped
 * from the free list when the position crosses a multiple of block_size) and this kernel
 * writes the token there ("PagedAttention and KV Cache Management", section "How Block Paging
 * Operates During Generation").
 *   key, value    device, [num_tokens][num_kv_heads][head_dim], contiguous, 16-byte aligned.
 *   k_pool,v_pool device, ONE layer's K and V planes (kv_pool_layer), 16-byte aligned.
 *   slot_mapping  device int64 [num_tokens]; distinct slots. A slot >= num_blocks*block_size is
 *                 skipped like a negative one (nothing is written outside the layer's region).
 * num_tokens == 0 is a no-op returning PKV_OK.
 */
pkv_status reshape_and_cache(const void* key, const void* value, void* k_pool, void* v_pool,
                             const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                             int head_dim, int block_size, int num_blocks, pkv_dtype dtype,
                             hipStream_t stream);

/*
 * reshape_and_cache into fp8 pools: for every token i with slot_mapping[i] >= 0, kv head h and
 * dim d, the K code at (slot / block_size, h, slot % block_size, d) becomes
 *     e4m3(fl32(key[i][h][d] * fl32(1 / k_scale)))      (V likewise with v_scale),
 * where e4m3 rounds to the nearest OCP E4M3 value (ties to even), saturates at +-448, and keeps
 * NaN and the sign of zero. Quantizing the cache to 8 bits halves its bytes ("KV-Cache
 * Management and PagedAttention", section "Planning capacity when context gets long"; "PagedAttention
 * and KV Cache Management", section "The KV Cache Size Equation"); the format and the per-pool
 * scale are this library's choice.
 *   key, value    device, [num_tokens][num_kv_heads][head_dim] of src_dtype (bf16 or fp16).
 *   k_pool,v_pool device, ONE layer's fp8 K and V planes (1 byte per element, layout above).
 *   k_scale, v_scale  finite, > 0.
 * Otherwise as reshape_and_cache.
 */
pkv_status reshape_and_cache_fp8(const void* key, const void* value, void* k_pool, void* v_pool,
                                 const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                                 int head_dim, int block_size, int num_blocks, pkv_dtype src_dtype,
                                 float k_scale, float v_scale, hipStream_t stream);

/*
 * Workgroups paged_attention_decode launches when it is passed num_workgroups == 0: one per 64
 * block positions (sequences x kv heads x head tiles x blocks of max_context_len), but at least
 * one per stream, and at most two per compute unit of the current device. The decode lays every
 * (sequence, kv head) stream of blocks end to end and gives each workgroup a contiguous share
 * (equal, or weighted by the XCD it runs on), so long and skewed sequences are spread evenly; a
 * stream cut between workgroups is joined by a log-sum-exp merge of fp32 partial results.
 * Returns 0 on invalid arguments.
 */
int paged_attention_num_workgroups(int num_seqs, int num_q_heads, int num_kv_heads,
                                   int max_context_len, int block_size);

/*
 * Workspace bytes paged_attention_decode needs for these arguments. The workspace holds the
 * partial softmax state of sequences whose blocks are split between workgroups ("PagedAttention
 * and KV Cache Management", section "Under the Hood: The PagedAttention CUDA Kernel": slices of
 * a sequence's logical blocks are processed separately and their softmax reductions combined
 * into one output). With G workgroups
 * (num_workgroups, or the library's choice when it is 0),
 *     bytes = G * 2 * 16 * (head_dim + 2) * 4 + roundup(4 G, 256)
 * (fp32 partials of at most two split streams per workgroup, then G arrival counters).
 * Returns (size_t)-1 on invalid arguments.
 */
size_t paged_attention_workspace_bytes(int num_seqs, int num_q_heads, int num_kv_heads,
                                       int head_dim, int block_size, int max_context_len,
                                       int num_workgroups);

/*
 * Decode attention over a paged KV cache. For each sequence s, query head h, kv head
 * g = h / (num_q_heads / num_kv_heads) and n = context_lens[s]:
 *     K_s[t] = K_pool[block_tables[s][t / B]][g][t % B][:],  t in [0, n)   (V_s likewise)
 *     x_t = scale * <q[s][h], K_s[t]>
 *     out[s][h] = sum_t exp(x_t - max_u x_u) V_s[t] / sum_t exp(x_t - max_u x_u)
 * ("KV-Cache Management and PagedAttention", section "Why the cache exists, and why it's so
 * hungry": each new token attends to every cached token; "PagedAttention and KV Cache
 * Management", section "Under the Hood: The PagedAttention CUDA Kernel".)
 * n == 0 gives out[s][:] = 0. Slots t >= n of the last block and table entries past
 * ceil(n / B) are never used, whatever they hold (NaN included).
 *   out          device, [num_seqs][num_q_heads][head_dim], same dtype as q.
 *   q            device, [num_seqs][num_q_heads][head_dim], contiguous, 16-byte aligned.
 *   k_pool/v_pool ONE layer's K and V planes (kv_pool_layer), 16-byte aligned.
 *   block_tables device int32 [num_seqs][max_blocks_per_seq].
 *   context_lens device int32 [num_seqs], each in [0, min(max_context_len, max_blocks_per_seq*B)].
 *   scale        multiplies q.k before the softmax (usually 1/sqrt(head_dim)).
 *   num_workgroups 0 = library choice (paged_attention_num_workgroups), else the number of
 *                workgroups (1 .. 2^20); results depend on it only through rounding order.
 *                With the library's choice of a full grid (two per compute unit), a batch of at
 *                most that many (sequence, kv head, head tile) streams whose lengths do not split
 *                evenly over it runs on the first half of the grid (one per compute unit), which
 *                cuts half as many streams; the result is then that of num_workgroups = half.
 *   workspace    device, >= paged_attention_workspace_bytes(...) bytes, 256-byte aligned. Its
 *                last 4 G bytes are arrival counters and the rest is scratch. Zero-fill the whole
 *                buffer once before its first use; every call that completes leaves its counters
 *                zero again, so the buffer can serve any later call it is large enough for.
 *                Calls that may run concurrently need separate workspaces.
 * At most 2048 sequences per call (PKV_ERR_UNSUPPORTED above).
 * Errors: PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED, PKV_ERR_ALIGNMENT, PKV_ERR_WORKSPACE,
 * PKV_ERR_HIP. Deterministic: identical inputs give bit-identical outputs (split streams are
 * merged in a fixed order, whichever workgroup finishes last).
 */
pkv_status paged_attention_decode(void* out, const void* q, const void* k_pool, const void* v_pool,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  float scale, int num_q_heads, int num_kv_heads, int head_dim,
                                  int block_size, int num_seqs, int max_blocks_per_seq,
                                  int max_context_len, int num_workgroups, pkv_dtype dtype,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Copy-on-write block copies: for each i in [0, num_copies), block src_blocks[i] is copied to
 * block dst_blocks[i] in every layer of `pool` (K and V, all kv heads, all block_size token
 * slots: one contiguous region per layer), bit-exact. This is the device half of copy-on-write ("PagedAttention
 * and KV Cache Management" (blog.sejan.dev), section "Advanced Memory Sharing: Prefix Caching &
 * Copy-on-Write", part 2: a fresh block receives a copy of the shared block before the writer's
 * table points at it). Run it before the reshape_and_cache that writes into the copies.
 *   src_blocks, dst_blocks  int32 [num_copies], 4-byte aligned, in device memory or pinned host
 *                           memory (pageable memory is refused with PKV_ERR_INVALID_ARG). A pair
 *                           with an id outside [0, num_blocks) is skipped on the device. A destination must not
 *                           appear twice or also be a source (the order of the copies is not
 *                           defined).
 * num_copies in [0, 65535]; 0 is a no-op.
 */
pkv_status copy_blocks(const pkv_pool* pool, const int32_t* src_blocks, const int32_t* dst_blocks,
                       int num_copies, hipStream_t stream);

/* Direction of swap_blocks. */
typedef enum { PKV_SWAP_OUT = 0, PKV_SWAP_IN = 1 } pkv_swap_dir;

/*
 * Swapping for preemption ("KV-Cache Management and PagedAttention", section "What paging unlocks
 * downstream", preemption and eviction; "PagedAttention and KV Cache Management", section
 * "Continuous Batching vs. Static Batching", preemption and GPU swapping): whole blocks move
 * between the device pool and a pool in host memory, K and V of every layer, bit-exact.
 *   PKV_SWAP_OUT: for each i, block src_blocks[i] of device_pool -> block dst_blocks[i] of
 *                 host_pool.
 *   PKV_SWAP_IN:  block src_blocks[i] of host_pool -> block dst_blocks[i] of device_pool.
 *   device_pool  a pool over device memory.
 *   host_pool    a pool created by kv_pool_create over PINNED host memory (hipHostMalloc, or a
 *                pinned torch tensor) with the same num_layers, num_kv_heads, head_dim,
 *                block_size and dtype as device_pool; its num_blocks may differ. Same layout.
 *   src_blocks, dst_blocks  int32 [num_pairs], 4-byte aligned, in device memory or pinned host
 *                memory (pageable memory is refused). A pair with an id outside its pool is
 *                skipped. Destinations must be
 *                distinct and must not be sources.
 * One kernel reads or writes the host pool across the host link, ordered on `stream`: synchronize
 * the stream before reading swapped-out blocks on the host, and do not write the host blocks of a
 * swap-in while it is in flight. Ids in device memory are read by that kernel, so they must be
 * written in stream order before it. A kernel that reaches into host memory starves work running
 * beside it on other streams: a decode slows several-fold for as long as the swap lasts. For swaps
 * that overlap a decode, use swap_blocks_dma. num_pairs in [0, 65535]; 0 is a no-op.
 * Errors: PKV_ERR_INVALID_ARG for null pools, mismatched geometry, a bad direction, or a host pool
 * or id array that is not device-visible (pinned host or device) memory, detected before any
 * launch.
 */
pkv_status swap_blocks(const pkv_pool* device_pool, const pkv_pool* host_pool,
                       const int32_t* src_blocks, const int32_t* dst_blocks, int num_pairs,
                       pkv_swap_dir direction, hipStream_t stream);

/*
 * swap_blocks on the GPU's copy engines instead of its compute units, for swaps that run while
 * other work (a decode step of the sequences still running) uses the GPU on another stream. The
 * same copies, directions and pool requirements as swap_blocks. Measured on MI355X, 2 sequences'
 * blocks of the 70B-shaped pool (16 layers, 512 MiB each way): about 37 GB/s, where swap_blocks
 * reaches about 56 GB/s. But a decode running beside it slows by 2-5%, where beside swap_blocks
 * it takes 80% longer.
 *   src_blocks, dst_blocks  int32 [num_pairs] in host memory (pinned or pageable), read during
 *                the call: the caller may reuse them once it returns.
 * Every id is checked before anything is enqueued: an id outside its pool refuses the whole call
 * with PKV_ERR_INVALID_ARG. The copies (one strided copy per block, its region in every layer)
 * are ordered on `stream`. Destinations must be distinct and must not be sources. The call costs
 * about 2 us of host time per block. num_pairs in [0, 65535]; 0 is a no-op.
 * Errors: PKV_ERR_INVALID_ARG (as swap_blocks, ids out of range, id arrays in device memory),
 * PKV_ERR_HIP if the runtime
 * refuses a copy (copies of earlier blocks may then already be enqueued).
 */
pkv_status swap_blocks_dma(const pkv_pool* device_pool, const pkv_pool* host_pool,
                           const int32_t* src_blocks, const int32_t* dst_blocks, int num_pairs,
                           pkv_swap_dir direction, hipStream_t stream);

/*
 * Host block manager: the bookkeeping of which physical blocks hold which sequence's tokens
 * ("PagedAttention and KV Cache Management" (blog.sejan.dev), sections "How Block Paging Operates
 * During Generation" (on-demand and boundary allocation), "Advanced Memory Sharing: Prefix Caching
 * & Copy-on-Write" (fork by reference counts, copy-on-write) and "Hands-On Implementation:
 * Building a PagedAttention Block Allocator in Python" (free blocks are handed out from the front
 * of the free list and returned to its back; running out is an error)).
 * It works on host memory only. A decode step calls kv_block_manager_append for its new tokens,
 * then copy_blocks of the returned pairs, reshape_and_cache into the returned slots, and
 * paged_attention_decode with the tables of kv_block_manager_tables. Sequences are named by
 * caller-chosen int64 ids. Every call succeeds completely or changes nothing. An object is not
 * thread-safe: one caller at a time.
 */
typedef struct pkv_block_manager pkv_block_manager;

/* A manager of num_blocks device blocks and num_host_blocks host blocks (for swapping; may be 0)
 * of block_size tokens, all free (free lists 0, 1, 2, ...). */
pkv_status kv_block_manager_create(pkv_block_manager** out, int num_blocks, int num_host_blocks,
                                   int block_size);
void kv_block_manager_destroy(pkv_block_manager* bm);  /* NULL is a no-op */
/* Free device blocks / free host blocks, or -1 for NULL. */
int kv_block_manager_num_free(const pkv_block_manager* bm);
int kv_block_manager_num_free_host(const pkv_block_manager* bm);

/* New sequence seq_id holding a prompt of num_tokens tokens: ceil(num_tokens / block_size)
 * blocks taken from the front of the free list. PKV_ERR_INVALID_ARG if seq_id exists,
 * PKV_ERR_NO_BLOCKS if the free list is too short. */
pkv_status kv_block_manager_allocate(pkv_block_manager* bm, int64_t seq_id, int64_t num_tokens);

/* New sequence dst_seq_id sharing every block (and the token count) of src_seq_id; each shared
 * block's reference count grows by one. No block is taken or copied. */
pkv_status kv_block_manager_fork(pkv_block_manager* bm, int64_t src_seq_id, int64_t dst_seq_id);

/*
 * One new token for each of seq_ids[0..num_seqs) (in order; an id may repeat). For token i,
 * slot_mapping[i] receives its slot (block * block_size + offset). A token that starts a new
 * logical block takes a block from the free list. A token written into a block that other
 * sequences still reference takes a fresh block; the pair (shared block, fresh block) is
 * appended to copy_src / copy_dst (host arrays of capacity num_seqs), and *num_copies is set to
 * the number of pairs. PKV_ERR_NO_BLOCKS (and no change at all) if the batch needs more blocks
 * than are free; PKV_ERR_INVALID_ARG for an unknown id.
 */
pkv_status kv_block_manager_append(pkv_block_manager* bm, const int64_t* seq_ids, int num_seqs,
                                   int64_t* slot_mapping, int32_t* copy_src, int32_t* copy_dst,
                                   int* num_copies);

/* The sequence ends: each of its blocks loses one reference; blocks at zero go to the back of
 * the free list, in table order (the host free list for a swapped-out sequence). */
pkv_status kv_block_manager_release(pkv_block_manager* bm, int64_t seq_id);

/*
 * Preemption by swapping ("KV-Cache Management and PagedAttention", section "What paging unlocks
 * downstream"; "PagedAttention and KV Cache Management", section "Continuous Batching vs. Static
 * Batching"): the group seq_ids[0..num_seqs) (distinct, all on the device) moves to host blocks.
 * Every distinct block of the group's tables, in order of first appearance (sequences in the
 * given order, tables in logical order), takes one host block from the front of the host free
 * list; pair k is (device_blocks[k] -> host_blocks[k]), *num_pairs pairs in host arrays of
 * capacity max_pairs. Then each table entry drops its reference on its device block (blocks at
 * zero go to the back of the free list, in that order) and points at the host block, so blocks
 * shared inside the group stay shared. Run swap_blocks(PKV_SWAP_OUT) of the pairs before any
 * freed device block is written again. A swapped-out sequence cannot be appended to, forked or
 * passed to kv_block_manager_tables; it can be released or swapped in.
 * PKV_ERR_NO_BLOCKS if the host free list is too short; PKV_ERR_INVALID_ARG for an unknown,
 * repeated or already swapped-out id or too small a capacity. Nothing changes on an error.
 */
pkv_status kv_block_manager_swap_out(pkv_block_manager* bm, const int64_t* seq_ids, int num_seqs,
                                     int32_t* device_blocks, int32_t* host_blocks, int max_pairs,
                                     int* num_pairs);

/* The reverse of kv_block_manager_swap_out for a group of swapped-out sequences: pairs
 * (host_blocks[k] -> device_blocks[k]) with device blocks from the front of the free list; run
 * swap_blocks(PKV_SWAP_IN) of the pairs before decoding the group. PKV_ERR_NO_BLOCKS if the
 * device free list is too short. */
pkv_status kv_block_manager_swap_in(pkv_block_manager* bm, const int64_t* seq_ids, int num_seqs,
                                    int32_t* host_blocks, int32_t* device_blocks, int max_pairs,
                                    int* num_pairs);

/*
 * Decode inputs for seq_ids[0..num_seqs): row i of block_tables (host int32
 * [num_seqs][max_blocks_per_seq]) receives sequence i's physical blocks, padded with -1, and
 * context_lens[i] its token count. PKV_ERR_INVALID_ARG (nothing written) for an unknown or
 * swapped-out id or a table longer than max_blocks_per_seq.
 */
pkv_status kv_block_manager_tables(const pkv_block_manager* bm, const int64_t* seq_ids,
                                   int num_seqs, int max_blocks_per_seq, int32_t* block_tables,
                                   int32_t* context_lens);

/*
 * paged_attention_decode over fp8 pools: as paged_attention_decode, with the key and value of a
 * slot taken as e4m3_value(code) * k_scale and e4m3_value(code) * v_scale. q and out are dtype
 * (bf16 or fp16); the pools hold E4M3 codes (PKV_FP8_E4M3 layout above). Accumulation is fp32;
 * key codes are widened exactly to dtype for the scores and value codes exactly to fp16 for the
 * weighted sum, whose softmax weights enter as one fp16 value (relative error at most 2^-12);
 * k_scale is applied to the scores and v_scale to the normalised output. Workspace and errors as paged_attention_decode;
 * k_scale, v_scale must be finite and > 0.
 */
pkv_status paged_attention_decode_fp8(void* out, const void* q, const void* k_pool,
                                      const void* v_pool, const int32_t* block_tables,
                                      const int32_t* context_lens, float scale, float k_scale,
                                      float v_scale, int num_q_heads, int num_kv_heads,
                                      int head_dim, int block_size, int num_seqs,
                                      int max_blocks_per_seq, int max_context_len,
                                      int num_workgroups, pkv_dtype dtype, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/*
 * One decode step fused into one launch: the same result as reshape_and_cache of each sequence's
 * newest token followed by paged_attention_decode ("PagedAttention and KV Cache Management"
 * (blog.sejan.dev), section "How Block Paging Operates During Generation": each step appends one
 * token per sequence, then attends over the whole context).
 *   key, value   device, [num_seqs][num_kv_heads][head_dim] of dtype: row s is the K / V of
 *                sequence s's token at position context_lens[s] - 1, the step's new token.
 *                Ignored for sequences with context length 0.
 *   k_pool, v_pool  one layer's K and V planes; the new token is written into its slot
 *                (block_tables[s][(n - 1) / block_size] * block_size + (n - 1) % block_size,
 *                bit-exact as reshape_and_cache writes it) by the workgroup that reads that
 *                slot's tile, before it reads anything, and then attended to like every other
 *                cached token.
 * context_lens and max_context_len count the new token. Everything else (layout, workspace,
 * errors, block-table trust) as paged_attention_decode. No other sequence may read or share the
 * blocks written here (copy-on-write has already made them private).
 */
pkv_status paged_attention_decode_append(void* out, const void* q, const void* key,
                                         const void* value, void* k_pool, void* v_pool,
                                         const int32_t* block_tables, const int32_t* context_lens,
                                         float scale, int num_q_heads, int num_kv_heads,
                                         int head_dim, int block_size, int num_seqs,
                                         int max_blocks_per_seq, int max_context_len,
                                         int num_workgroups, pkv_dtype dtype, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream);

/* paged_attention_decode_append over fp8 pools: the new token is quantized as
 * reshape_and_cache_fp8 does (k_scale, v_scale), written into the pool, and attended to through
 * the values of its codes, as paged_attention_decode_fp8 would read them back. */
pkv_status paged_attention_decode_append_fp8(void* out, const void* q, const void* key,
                                             const void* value, void* k_pool, void* v_pool,
                                             const int32_t* block_tables,
                                             const int32_t* context_lens, float scale,
                                             float k_scale, float v_scale, int num_q_heads,
                                             int num_kv_heads, int head_dim, int block_size,
                                             int num_seqs, int max_blocks_per_seq,
                                             int max_context_len, int num_workgroups,
                                             pkv_dtype dtype, void* workspace,
                                             size_t workspace_bytes, hipStream_t stream);

/*
 * Bytes of the library's own decode scratch on each device (see paged_attention_decode_noalloc):
 * the workspace of 1024 workgroups at head_dim 128.
 */
#define PKV_NOALLOC_SCRATCH_BYTES 17043456

/*
 * paged_attention_decode for callers that cannot allocate device memory: code being captured
 * into a HIP graph, tight serving loops, harnesses that forbid hipMalloc. Same arguments, result
 * and errors as paged_attention_decode (16-bit pools), but no workspace argument: the split-stream
 * partials and arrival counters live in a static device array of PKV_NOALLOC_SCRATCH_BYTES bytes
 * that the library holds on each device it runs on until the process ends. The call allocates
 * nothing (no hipMalloc, no library allocation) and does not synchronise.
 *   - Limit: paged_attention_workspace_bytes(...) for these arguments (with the library's grid
 *     choice when num_workgroups is 0) must not exceed PKV_NOALLOC_SCRATCH_BYTES, i.e. at most
 *     1024 workgroups at head_dim 128 (about 2000 at 64); larger requests return
 *     PKV_ERR_WORKSPACE and launch nothing. The library's default grid (two workgroups per compute
 *     unit) always fits on MI355X.
 *   - The first call on a device looks up the array's device address and clears its arrival
 *     counters with a small kernel on `stream`; every completed call leaves them zero again.
 *   - All calls on one device share the one array: calls that may overlap in time on the same
 *     device (different streams, or one graph replayed concurrently with another call) race and
 *     give wrong results. Calls ordered on one stream are safe.
 * Returns PKV_ERR_HIP if the array cannot be located on the current device.
 */
pkv_status paged_attention_decode_noalloc(void* out, const void* q, const void* k_pool,
                                          const void* v_pool, const int32_t* block_tables,
                                          const int32_t* context_lens, float scale,
                                          int num_q_heads, int num_kv_heads, int head_dim,
                                          int block_size, int num_seqs, int max_blocks_per_seq,
                                          int max_context_len, int num_workgroups,
                                          pkv_dtype dtype, hipStream_t stream);

/*
 * Debug check of a step's index inputs, on the device, reading nothing but them (never the pool,
 * so it is safe on the very inputs it is meant to catch). The decode and scatter kernels trust
 * these indices: a sequence's table must name pool blocks that hold its tokens ("PagedAttention
 * and KV Cache Management", section "PagedAttention: OS Virtual Memory Architecture for GPUs"),
 * and every new token owns one slot ("How Block Paging Operates During Generation").
 * Counts, written to result (device int32 [4], 4-byte aligned):
 *   result[0]  used table entries outside [0, num_blocks): block_tables[s][j] for
 *              j < ceil(n / block_size), n = context_lens[s] clamped to
 *              [0, max_blocks_per_seq * block_size] as the decode clamps it;
 *   result[1]  context lengths outside [0, min(max_context_len, max_blocks_per_seq * block_size)];
 *   result[2]  slots equal to an earlier non-negative slot of slot_mapping (repeats);
 *   result[3]  slots at or past num_blocks * block_size (reshape_and_cache skips them).
 *   block_tables device int32 [num_seqs][max_blocks_per_seq]; context_lens device int32
 *                [num_seqs]; slot_mapping device int64 [num_tokens], or NULL with
 *                num_tokens == 0.
 * The counts are written by kernels on `stream`: read them once it has finished. The repeat
 * count compares each slot with every earlier one (quadratic in num_tokens; the earlier slots are
 * staged through LDS in tiles of 256). On MI355X a 64-sequence decode step's inputs take about
 * 6 us, and a prefill of 16,384 slots about 0.5 ms. It is a debug aid, not meant for every step
 * of a serving loop.
 * Errors: PKV_ERR_INVALID_ARG (negative sizes, num_blocks or block_size < 1, NULL where data is
 * read: context_lens when num_seqs > 0, block_tables when there are table entries, slot_mapping
 * when num_tokens > 0), PKV_ERR_UNSUPPORTED (sizes past 32-bit indexing), PKV_ERR_ALIGNMENT,
 * PKV_ERR_HIP.
 */
pkv_status paged_attention_check_inputs(const int32_t* block_tables, const int32_t* context_lens,
                                        int num_seqs, int max_blocks_per_seq, int max_context_len,
                                        int block_size, int num_blocks,
                                        const int64_t* slot_mapping, int num_tokens,
                                        int32_t* result, hipStream_t stream);

/* Static, human-readable name of a status code. */
const char* pkv_status_string(pkv_status status);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H_ */
