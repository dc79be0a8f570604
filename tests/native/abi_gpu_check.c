/* The decode path driven from plain C, with no Python or PyTorch: device memory from hipMalloc,
 * a one-layer bf16 pool described by kv_pool_create, every token's key and value scattered by
 * reshape_and_cache, then paged_attention_decode with the library's choice of grid, and
 * paged_attention_check_inputs of the same inputs (all counts zero). Four
 * sequences of 1, 15, 16 and 41 tokens; the 41-token one uses the page's block table [7, 3, 9]
 * ("KV-Cache Management and PagedAttention", section "PagedAttention: treat the cache like
 * virtual memory"). Inputs come from a fixed linear congruential generator. The program writes
 * its inputs, the pool after the scatter and the decode output to the file named on the command
 * line; the test checks them against the oracle. */
#include "pagedkv.h"

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

enum { S = 4, HQ = 8, HKV = 2, D = 64, B = 16, NB = 64, MAXB = 3, MAXCTX = 41 };
static const int32_t kLens[S] = {1, 15, 16, 41};
static const int32_t kTables[S][MAXB] = {{12, -1, -1}, {5, -1, -1}, {40, -1, -1}, {7, 3, 9}};

static uint32_t lcg_state = 12345u;
static float next_uniform(void) { /* in [-1, 1) */
  lcg_state = lcg_state * 1664525u + 1013904223u;
  return (float)(lcg_state >> 8) / 16777216.0f * 2.0f - 1.0f;
}
static uint16_t bf16_bits(float x) { /* round to nearest even (finite x) */
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

#define HIP_CHECK(call)                                                      \
  do {                                                                       \
    hipError_t e_ = (call);                                                  \
    if (e_ != hipSuccess) {                                                  \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));      \
      return 2;                                                              \
    }                                                                        \
  } while (0)
#define PKV_CHECK(call)                                                      \
  do {                                                                       \
    pkv_status s_ = (call);                                                  \
    if (s_ != PKV_OK) {                                                      \
      fprintf(stderr, "%s failed: %s\n", #call, pkv_status_string(s_));      \
      return 3;                                                              \
    }                                                                        \
  } while (0)

int main(int argc, char** argv) {
  if (argc != 2) {
    fprintf(stderr, "usage: %s OUTPUT_FILE\n", argv[0]);
    return 1;
  }
  int T = 0;
  for (int s = 0; s < S; ++s) T += kLens[s];
  int64_t* slots = malloc(sizeof(int64_t) * T);
  uint16_t* key = malloc(sizeof(uint16_t) * T * HKV * D);
  uint16_t* val = malloc(sizeof(uint16_t) * T * HKV * D);
  uint16_t q[S * HQ * D], out[S * HQ * D];
  if (!slots || !key || !val) return 1;
  for (int s = 0, i = 0; s < S; ++s)
    for (int t = 0; t < kLens[s]; ++t, ++i) slots[i] = (int64_t)kTables[s][t / B] * B + t % B;
  for (int i = 0; i < T * HKV * D; ++i) key[i] = bf16_bits(next_uniform());
  for (int i = 0; i < T * HKV * D; ++i) val[i] = bf16_bits(next_uniform());
  for (int i = 0; i < S * HQ * D; ++i) q[i] = bf16_bits(next_uniform());

  const size_t pool_bytes = kv_pool_bytes(1, NB, HKV, D, B, PKV_BF16);
  const size_t ws_bytes = paged_attention_workspace_bytes(S, HQ, HKV, D, B, MAXCTX, 0);
  if (pool_bytes == 0 || ws_bytes == 0) return 1;
  void *d_pool, *d_ws, *d_key, *d_val, *d_q, *d_out, *d_slots, *d_tables, *d_lens;
  HIP_CHECK(hipMalloc(&d_pool, pool_bytes));
  HIP_CHECK(hipMalloc(&d_ws, ws_bytes));
  HIP_CHECK(hipMalloc(&d_key, sizeof(uint16_t) * T * HKV * D));
  HIP_CHECK(hipMalloc(&d_val, sizeof(uint16_t) * T * HKV * D));
  HIP_CHECK(hipMalloc(&d_q, sizeof q));
  HIP_CHECK(hipMalloc(&d_out, sizeof out));
  HIP_CHECK(hipMalloc(&d_slots, sizeof(int64_t) * T));
  HIP_CHECK(hipMalloc(&d_tables, sizeof kTables));
  HIP_CHECK(hipMalloc(&d_lens, sizeof kLens));
  HIP_CHECK(hipMemset(d_pool, 0, pool_bytes));
  HIP_CHECK(hipMemset(d_ws, 0, ws_bytes));
  HIP_CHECK(hipMemcpy(d_key, key, sizeof(uint16_t) * T * HKV * D, hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(d_val, val, sizeof(uint16_t) * T * HKV * D, hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(d_q, q, sizeof q, hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(d_slots, slots, sizeof(int64_t) * T, hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(d_tables, kTables, sizeof kTables, hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(d_lens, kLens, sizeof kLens, hipMemcpyHostToDevice));

  pkv_pool* pool = NULL;
  void *k_layer, *v_layer;
  PKV_CHECK(kv_pool_create(&pool, d_pool, pool_bytes, 1, NB, HKV, D, B, PKV_BF16));
  PKV_CHECK(kv_pool_layer(pool, 0, &k_layer, &v_layer));
  PKV_CHECK(reshape_and_cache(d_key, d_val, k_layer, v_layer, (const int64_t*)d_slots, T, HKV, D,
                              B, NB, PKV_BF16, 0));
  PKV_CHECK(paged_attention_decode(d_out, d_q, k_layer, v_layer, (const int32_t*)d_tables,
                                   (const int32_t*)d_lens, 1.0f / sqrtf((float)D), HQ, HKV, D, B,
                                   S, MAXB, MAXCTX, 0, PKV_BF16, d_ws, ws_bytes, 0));
  /* The debug check of the same inputs: clean, so every count is zero. */
  void* d_counts;
  int32_t counts[4] = {-1, -1, -1, -1};
  HIP_CHECK(hipMalloc(&d_counts, sizeof counts));
  PKV_CHECK(paged_attention_check_inputs((const int32_t*)d_tables, (const int32_t*)d_lens, S, MAXB,
                                         MAXCTX, B, NB, (const int64_t*)d_slots, T,
                                         (int32_t*)d_counts, 0));
  HIP_CHECK(hipDeviceSynchronize());
  HIP_CHECK(hipMemcpy(counts, d_counts, sizeof counts, hipMemcpyDeviceToHost));
  HIP_CHECK(hipFree(d_counts));
  if (counts[0] || counts[1] || counts[2] || counts[3]) {
    fprintf(stderr, "input check counted %d %d %d %d\n", counts[0], counts[1], counts[2],
            counts[3]);
    return 4;
  }
  HIP_CHECK(hipMemcpy(out, d_out, sizeof out, hipMemcpyDeviceToHost));
  unsigned char* pool_host = malloc(pool_bytes);
  if (!pool_host) return 1;
  HIP_CHECK(hipMemcpy(pool_host, d_pool, pool_bytes, hipMemcpyDeviceToHost));

  FILE* f = fopen(argv[1], "wb");
  if (!f) return 1;
  const int32_t header[9] = {S, HQ, HKV, D, B, NB, MAXB, MAXCTX, T};
  fwrite(header, sizeof header, 1, f);
  fwrite(kLens, sizeof kLens, 1, f);
  fwrite(kTables, sizeof kTables, 1, f);
  fwrite(slots, sizeof(int64_t), T, f);
  fwrite(q, sizeof q, 1, f);
  fwrite(key, sizeof(uint16_t), T * HKV * D, f);
  fwrite(val, sizeof(uint16_t), T * HKV * D, f);
  fwrite(out, sizeof out, 1, f);
  fwrite(pool_host, 1, pool_bytes, f);
  fclose(f);

  kv_pool_destroy(pool);
  hipFree(d_pool); hipFree(d_ws); hipFree(d_key); hipFree(d_val); hipFree(d_q); hipFree(d_out);
  hipFree(d_slots); hipFree(d_tables); hipFree(d_lens);
  free(slots); free(key); free(val); free(pool_host);
  printf("C decode done: %d tokens scattered, %d x %d rows decoded\n", T, S, HQ);
  return 0;
}
