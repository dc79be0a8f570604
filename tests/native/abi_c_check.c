/* The library's ABI used from plain C (compiled as C11 by gcc, linked against libpagedkv.so):
 * the header must be valid C, and the host-side entry points behave as the header states. Only
 * calls that touch no GPU: pool sizing, status strings, the host block manager, and the argument
 * refusals of swap_blocks_dma. */
#include "pagedkv.h"

#include <stdio.h>
#include <string.h>

static int failures = 0;
#define CHECK(cond)                                          \
  do {                                                       \
    if (!(cond)) {                                           \
      printf("FAIL line %d: %s\n", __LINE__, #cond);         \
      ++failures;                                            \
    }                                                        \
  } while (0)

int main(void) {
  /* Pool sizing: 2 (K, V) x layers x blocks x kv heads x block_size x head_dim x element bytes.
   * 80 layers, 8 kv heads, d128, 16-bit: 327,680 B per token ("PagedAttention and KV Cache
   * Management", section "Real-World Memory Sizing Example (LLaMA-3-70B)"), so one 16-token block
   * of every layer holds 16 times that. */
  CHECK(kv_pool_bytes(80, 1, 8, 128, 16, PKV_BF16) == (size_t)327680 * 16);
  CHECK(kv_pool_bytes(80, 16384, 8, 128, 16, PKV_BF16) == (size_t)85899345920ULL);
  CHECK(kv_pool_bytes(1, 1, 1, 128, 16, PKV_FP8_E4M3) == (size_t)2 * 16 * 128);
  CHECK(kv_pool_bytes(0, 1, 1, 128, 16, PKV_BF16) == 0);
  CHECK(kv_pool_bytes(1, 1, 1, 96, 16, PKV_BF16) == 0); /* no kernel for head_dim 96 */
  CHECK(pkv_status_string(PKV_OK) != NULL && strlen(pkv_status_string(PKV_OK)) > 0);
  CHECK(pkv_status_string(PKV_ERR_NO_BLOCKS) != NULL);

  /* Block manager: 8 device blocks of 4 tokens, free list 0, 1, ..., 7. */
  pkv_block_manager* bm = NULL;
  CHECK(kv_block_manager_create(&bm, 8, 0, 4) == PKV_OK && bm != NULL);
  if (bm == NULL) return 1;
  CHECK(kv_block_manager_num_free(bm) == 8);
  CHECK(kv_block_manager_allocate(bm, 1, 10) == PKV_OK); /* ceil(10 / 4) = 3 blocks: 0, 1, 2 */
  CHECK(kv_block_manager_num_free(bm) == 5);
  CHECK(kv_block_manager_fork(bm, 1, 2) == PKV_OK); /* shares 0, 1, 2; takes nothing */
  CHECK(kv_block_manager_num_free(bm) == 5);

  /* Token 10 of sequence 2 lands at offset 10 % 4 = 2 of its third block, which sequence 1 still
   * references: copy-on-write into the next free block, 3. */
  int64_t ids[1] = {2};
  int64_t slot = -1;
  int32_t src[1] = {-1}, dst[1] = {-1};
  int ncopy = -1;
  CHECK(kv_block_manager_append(bm, ids, 1, &slot, src, dst, &ncopy) == PKV_OK);
  CHECK(ncopy == 1 && src[0] == 2 && dst[0] == 3);
  CHECK(slot == 3 * 4 + 2);
  CHECK(kv_block_manager_num_free(bm) == 4);

  int64_t both[2] = {1, 2};
  int32_t tables[2 * 4];
  int32_t lens[2];
  CHECK(kv_block_manager_tables(bm, both, 2, 4, tables, lens) == PKV_OK);
  CHECK(lens[0] == 10 && lens[1] == 11);
  CHECK(tables[0] == 0 && tables[1] == 1 && tables[2] == 2 && tables[3] == -1);
  CHECK(tables[4] == 0 && tables[5] == 1 && tables[6] == 3 && tables[7] == -1);

  /* 100 tokens need 25 blocks with 4 free: refused, nothing taken. */
  CHECK(kv_block_manager_allocate(bm, 3, 100) == PKV_ERR_NO_BLOCKS);
  CHECK(kv_block_manager_num_free(bm) == 4);
  /* Sequence 1 ends: block 2, which only it still referenced, returns; 0 and 1 stay with 2. */
  CHECK(kv_block_manager_release(bm, 1) == PKV_OK);
  CHECK(kv_block_manager_num_free(bm) == 5);

  kv_block_manager_destroy(bm);
  kv_block_manager_destroy(NULL);
  printf("C ABI checks: failures %d\n", failures);
  /* swap_blocks_dma: its argument refusals come before any HIP call (pools here describe a host
   * arena; nothing is copied). */
  static unsigned char arena[4096] __attribute__((aligned(256)));
  pkv_pool* pa = NULL;
  pkv_pool* pb = NULL;
  CHECK(kv_pool_create(&pa, arena, sizeof arena, 1, 1, 1, 64, 16, PKV_FP8_E4M3) == PKV_OK);
  CHECK(kv_pool_create(&pb, arena, sizeof arena, 1, 1, 1, 128, 16, PKV_FP8_E4M3) == PKV_OK);
  int32_t one[1] = {0};
  CHECK(swap_blocks_dma(NULL, pa, one, one, 1, PKV_SWAP_OUT, NULL) == PKV_ERR_INVALID_ARG);
  CHECK(swap_blocks_dma(pa, pa, one, one, 1, (pkv_swap_dir)7, NULL) == PKV_ERR_INVALID_ARG);
  CHECK(swap_blocks_dma(pa, pb, one, one, 1, PKV_SWAP_OUT, NULL) == PKV_ERR_INVALID_ARG);
  CHECK(swap_blocks_dma(pa, pa, one, one, -1, PKV_SWAP_OUT, NULL) == PKV_ERR_INVALID_ARG);
  CHECK(swap_blocks_dma(pa, pa, NULL, NULL, 0, PKV_SWAP_IN, NULL) == PKV_OK); /* no-op */
  kv_pool_destroy(pa);
  kv_pool_destroy(pb);

  return failures != 0;
}
