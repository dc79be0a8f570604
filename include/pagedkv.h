/*
 * pagedkv.h — C ABI of libpagedkv: PagedAttention decode on AMD Instinct MI355X (gfx950).
 *
 * The library implements the decode step of paged attention. A sequence's keys and values live in
 * fixed-size blocks of `block_size` tokens, scattered over one shared physical block pool; a
 * per-sequence block table maps logical block j (tokens j*B .. j*B+B-1) to a physical block id.
 * The attention kernel takes the block table as an argument and gathers K and V through it in
 * place, with no staging copy into contiguous memory.
 *   - "KV-Cache Management and PagedAttention" (adversariallm.ai), section
 *     "PagedAttention: treat the cache like virtual memory" (block table, block size 16,
 *     the tok 0..40 -> phys [7,3,9] diagram).
 *   - "PagedAttention and KV Cache Management" (blog.sejan.dev), sections
 *     "PagedAttention: OS Virtual Memory Architecture for GPUs" (physical pool, block table),
 *     "How Block Paging Operates During Generation" (boundary allocation; block byte size spans
 *     all layers) and "Under the Hood: The PagedAttention CUDA Kernel"
 *     (physical_block_id = block_table[seq_id, logical_block_id]; softmax over the gathered keys).
 *
 * Conventions for every entry point
 *   - Device pointers are HIP device addresses owned by the caller. The library never allocates
 *     or frees device memory. A `pkv_pool` object holds host-side geometry only.
 *   - Calls that take a `stream` enqueue their kernels on it and return without synchronising.
 *     A NULL stream is the HIP null stream.
 *   - Argument errors found on the host come back as a negative `pkv_status` and nothing is
 *     launched. A failed kernel launch returns PKV_ERR_HIP. Nothing is thrown across the ABI.
 *   - Device-resident indices (block table entries, context lengths, slots) are NOT validated:
 *     block ids must lie in [0, num_blocks), context lengths in [0, max_context_len] and
 *     [0, max_blocks_per_seq*block_size], and slots must be distinct within one call.
 *     Violations are undefined behaviour (out-of-bounds device accesses).
 *   - Stateless and thread-safe: concurrent calls are fine as long as their outputs do not alias.
 *
 * Element types: bf16 (PKV_BF16) or IEEE fp16 (PKV_FP16); q, key, value, the pools and out all use
 * the same type. Accumulation is fp32.
 *
 * Supported shapes: head_dim in {64, 128}; block_size == 16; num_q_heads % num_kv_heads == 0
 * (query head h reads kv head h / (num_q_heads / num_kv_heads): consecutive query heads form one
 * group); any group size.
 *
 * ---------------------------------------------------------------------------------------------
 * KV pool layout (the one data format this ABI defines)
 *
 * K and V are two separate pools of 16-bit elements. Element (layer L, block b, kv head h,
 * token slot t in [0,B), dim d in [0,D)) lives at element index
 *
 *     ((L * num_blocks + b) * num_kv_heads + h) * (B * D) + tile_offset(t, d)
 *
 * i.e. the pool is [layer][block][kv_head][tile], one tile = B*D elements (4 KiB for D=128, B=16)
 * and tile bases are 4 KiB aligned when the pool base is. Inside a tile, the B tokens are split
 * into sub-tiles of 16 tokens (sub = t / 16, u = t % 16), each 16*D elements; within a sub-tile:
 *
 *   K tile:  k_off(u, d) = (d / 8) * 128 + u * 8 + (d % 8)
 *            -> [D/8][16 tokens][8 dims]: eight consecutive dims of one token are one 16-byte
 *               chunk, and the 16 tokens' chunks for the same eight dims are contiguous.
 *   V tile:  v_off(u, d) = ((((d / 32) * 4 + u / 4) * 16 + d % 16) * 2 + (d / 16) % 2) * 4 + u % 4
 *            -> [D/32][4 token quads][16 dims][2 dim halves][4 tokens]: four consecutive tokens of
 *               one dim are one 8-byte chunk.
 *   tile_offset(t, d) = (t / 16) * 16 * D + {k_off | v_off}(t % 16, d)
 *
 * Worked examples (D = 128, B = 16): K (t=1,d=0) -> 8; K (t=0,d=8) -> 128; K (t=5,d=37) -> 557;
 * V (t=1,d=0) -> 1; V (t=0,d=1) -> 8; V (t=0,d=16) -> 4; V (t=5,d=37) -> 681;
 * V (t=15,d=127) -> 2047.
 * With these layouts one wavefront reads a whole K or V tile as 64 lanes x 16 bytes per load
 * instruction, every instruction covering one contiguous, 1 KiB aligned range, and each lane's
 * 16 bytes are already the operand of one gfx950 matrix-core instruction.
 *
 * A slot is `physical_block * block_size + t` (token slot t of that block).
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
  PKV_ERR_HIP = -5          /* the HIP runtime reported an error at launch */
} pkv_status;

typedef enum { PKV_BF16 = 0, PKV_FP16 = 1 } pkv_dtype;

/* Opaque host-side description of one K pool and one V pool holding every layer. */
typedef struct pkv_pool pkv_pool;

/*
 * Bytes of ONE of the two pools (K or V) for all layers:
 *   num_layers * num_blocks * num_kv_heads * block_size * head_dim * 2.
 * This is the per-token KV size of the sizing formula ("KV-Cache Management and PagedAttention",
 * section "Why the cache exists, and why it's so hungry"; "PagedAttention and KV Cache
 * Management", section "The KV Cache Size Equation"), halved because K and V are separate pools,
 * times block_size * num_blocks tokens. Returns 0 for any non-positive argument, an
 * unsupported shape, or on size_t overflow.
 */
size_t kv_pool_bytes(int num_layers, int num_blocks, int num_kv_heads, int head_dim, int block_size,
                     pkv_dtype dtype);

/*
 * Describe caller-allocated K and V pools (device memory, `bytes_each` bytes each, laid out as
 * above). Checks: non-NULL, 256-byte aligned bases, bytes_each >= kv_pool_bytes(...), supported
 * shape. On success *out receives a new host object (free it with kv_pool_destroy). The device
 * memory stays owned by the caller and must outlive the object. No device work is done.
 */
pkv_status kv_pool_create(pkv_pool** out, void* k_base, void* v_base, size_t bytes_each,
                          int num_layers, int num_blocks, int num_kv_heads, int head_dim,
                          int block_size, pkv_dtype dtype);

/* Device addresses of layer `layer`'s K and V sub-pools ([num_blocks][num_kv_heads][tile]). */
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
 *   k_pool,v_pool device, ONE layer's sub-pool (kv_pool_layer), 16-byte aligned.
 *   slot_mapping  device int64 [num_tokens]; slots must be < num_blocks*block_size and distinct.
 * num_tokens == 0 is a no-op returning PKV_OK.
 */
pkv_status reshape_and_cache(const void* key, const void* value, void* k_pool, void* v_pool,
                             const int64_t* slot_mapping, int num_tokens, int num_kv_heads,
                             int head_dim, int block_size, int num_blocks, pkv_dtype dtype,
                             hipStream_t stream);

/*
 * Workgroups paged_attention_decode launches when it is passed num_workgroups == 0: enough to fill
 * every compute unit of the current device, fewer for small batches. The decode lays every
 * (sequence, kv head) stream of blocks end to end and gives each workgroup an equal contiguous
 * share, so long and skewed sequences are spread evenly; a stream cut between workgroups is
 * joined by a log-sum-exp merge of fp32 partial results. Returns 0 on invalid arguments.
 */
int paged_attention_num_workgroups(int num_seqs, int num_q_heads, int num_kv_heads,
                                   int max_context_len, int block_size);

/*
 * Workspace bytes paged_attention_decode needs for these arguments: with G workgroups
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
 *   k_pool/v_pool ONE layer's sub-pools (kv_pool_layer), 16-byte aligned.
 *   block_tables device int32 [num_seqs][max_blocks_per_seq].
 *   context_lens device int32 [num_seqs], each in [0, min(max_context_len, max_blocks_per_seq*B)].
 *   scale        multiplies q.k before the softmax (usually 1/sqrt(head_dim)).
 *   num_workgroups 0 = library choice (paged_attention_num_workgroups), else the number of
 *                workgroups (1 .. 2^20); results depend on it only through rounding order.
 *   workspace    device, >= paged_attention_workspace_bytes(...) bytes, 256-byte aligned. Its
 *                last 4 G bytes are arrival counters and the rest is scratch. Zero-fill the whole
 *                buffer once before its first use; every call that completes leaves its counters
 *                zero again, so the buffer can serve any later call it is large enough for.
 *                Calls that may run concurrently need separate workspaces.
 * At most 2048 sequences per call (PKV_ERR_UNSUPPORTED above).
 * Errors: PKV_ERR_INVALID_ARG, PKV_ERR_UNSUPPORTED, PKV_ERR_ALIGNMENT, PKV_ERR_WORKSPACE,
 * PKV_ERR_HIP. Deterministic: identical inputs give bit-identical outputs (no atomics).
 */
pkv_status paged_attention_decode(void* out, const void* q, const void* k_pool, const void* v_pool,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  float scale, int num_q_heads, int num_kv_heads, int head_dim,
                                  int block_size, int num_seqs, int max_blocks_per_seq,
                                  int max_context_len, int num_workgroups, pkv_dtype dtype,
                                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Static, human-readable name of a status code. */
const char* pkv_status_string(pkv_status status);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H_ */
