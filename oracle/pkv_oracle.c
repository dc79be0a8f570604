/*
 * pkv_oracle.c — CPU oracle for paged-attention decode and the reshape_and_cache scatter.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, plain reference that the GPU library is
 * checked against. Only the test-suite, the package smoke check and the benchmark's CPU-baseline
 * leg may build, load or call it; the product path never does. It shares no code, header, table
 * or helper with the HIP library: every formula below is written out again from its definition.
 *
 * Arithmetic: fp64 throughout, on the exact values of the 16-bit inputs (every bf16 and fp16
 * value is exactly representable as a double) and on the fp32 `scale` widened exactly.
 *
 * What it computes
 *   1. Gather ("PagedAttention and KV Cache Management" (blog.sejan.dev), section "Under the
 *      Hood: The PagedAttention CUDA Kernel": the kernel maps a sequence's logical block to
 *      its physical block through the table; "KV-Cache Management and PagedAttention"
 *      (adversariallm.ai), section "PagedAttention: treat the cache like virtual memory"):
 *      token t of sequence s is slot
 *      t mod B of physical block block_table[s][floor(t / B)]. The sequence's keys and values
 *      are reassembled into contiguous order K_c[t], V_c[t], t = 0 .. n-1 — the layout paging
 *      replaced ("PagedAttention and KV Cache Management", section "The Memory Fragmentation
 *      Crisis in Traditional Serving").
 *   2. Dense attention of one query over those rows ("KV-Cache Management and PagedAttention",
 *      section "Why the cache exists, and why it's so hungry": a decode step's query is scored
 *      against all cached keys of its sequence): x_t = scale * q.K_c[t]; m = max_t x_t; w_t = exp(x_t - m);
 *      out = sum_t w_t V_c[t] / sum_t w_t. Query head h reads kv head h / (Hq / Hkv)
 *      (grouped-query attention, "PagedAttention and KV Cache Management", section "The KV
 *      Cache Size Equation": n_kv_heads << n_q_heads; contiguous groups are this oracle's
 *      reading). n = 0 gives a zero output (a convention: the pages never reach that case).
 *   3. Scatter ("PagedAttention and KV Cache Management", section "How Block Paging Operates
 *      During Generation"): a new token whose slot is physical_block * B + t is written to
 *      slot t of that block, for every kv head; negative slots are skipped.
 *
 * Pool layout: the library's documented data format — [block][kv_head][tile] with the K and V
 * tile orders described in include/pagedkv.h — re-derived here in pool_index() (16-bit pools)
 * and pool_index8() (fp8 pools).
 *
 * fp8 KV ("KV-Cache Management and PagedAttention", section "Planning capacity when context gets
 * long", and "PagedAttention and KV Cache Management", section "The KV Cache Size Equation":
 * quantizing the cache to 8 bits halves dtype_bytes). The pages name no format or scaling;
 * the reading used here: OCP FP8 E4M3 ("e4m3fn": 1 sign, 4 exponent bits with bias 7, 3
 * mantissa bits, no infinities, S.1111.111 is NaN, largest finite 448), one fp32 scale per pool
 * (K and V), stored code = e4m3(fl32(x * fl32(1 / scale))) with round-to-nearest-even and
 * saturation to the largest finite value, and value = e4m3_value(code) * scale.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORACLE_BF16 = 0, ORACLE_FP16 = 1 };

/* bf16 is the upper half of an IEEE binary32: widen by appending 16 zero bits. */
static double bf16_value(uint16_t bits) {
  uint32_t w = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &w, sizeof f);
  return (double)f;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double fp16_value(uint16_t bits) {
  int sign = bits >> 15;
  int e = (bits >> 10) & 31;
  int f = bits & 1023;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24); /* subnormal: f * 2^-14 / 2^10 */
  } else if (e == 31) {
    v = f ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + f), e - 25); /* (1 + f/1024) * 2^(e-15) */
  }
  return sign ? -v : v;
}

static double elem_value(uint16_t bits, int dtype) {
  return dtype == ORACLE_FP16 ? fp16_value(bits) : bf16_value(bits);
}

/* OCP E4M3: value of an 8-bit code, from the format's definition. */
static double e4m3_value(uint8_t code) {
  int sign = code >> 7;
  int e = (code >> 3) & 15;
  int m = code & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0) {
    v = ldexp((double)m, -9); /* subnormal: (m / 8) * 2^-6 */
  } else {
    v = ldexp((double)(8 + m), e - 10); /* (1 + m/8) * 2^(e-7) */
  }
  return sign ? -v : v;
}

double oracle_e4m3_value(int code) { return e4m3_value((uint8_t)code); }

/*
 * Nearest E4M3 code to y: among the 127 non-negative finite codes, the one whose value is
 * closest to |y| (ties to the code with an even mantissa), with y's sign; |y| beyond the largest
 * finite value gives that value (saturation); NaN gives S.1111.111.
 */
static uint8_t e4m3_encode(float y) {
  uint8_t sign = signbit(y) ? 0x80 : 0x00;
  if (isnan(y)) return (uint8_t)(sign | 0x7F);
  double a = fabs((double)y);
  int best = 0;
  double best_err = INFINITY;
  for (int c = 0; c <= 0x7E; ++c) {
    double err = fabs(a - e4m3_value((uint8_t)c));
    if (err < best_err || (err == best_err && (c & 1) == 0)) {
      best = c;
      best_err = err;
    }
  }
  return (uint8_t)(sign | best);
}

int oracle_e4m3_encode(float y) { return e4m3_encode(y); }

/*
 * Element index of (block b, kv head h, token slot t, dim d) in one layer's K (is_v = 0) or
 * V (is_v = 1) pool. A tile of B*D elements per (block, kv head); inside it, sub-tiles of 16
 * tokens; inside a sub-tile, K is ordered [d/8][token][d%8] and V is ordered
 * [d/32][token/4][d%16][(d/16)%2][token%4].
 */
static size_t pool_index(int is_v, long b, int h, int t, int d, int Hkv, int B, int D) {
  size_t tile = ((size_t)b * (size_t)Hkv + (size_t)h) * (size_t)B * (size_t)D;
  int sub = t / 16;
  int u = t % 16;
  size_t within;
  if (!is_v) {
    within = (size_t)(d / 8) * 128 + (size_t)u * 8 + (size_t)(d % 8);
  } else {
    size_t dim_group = (size_t)(d / 32);
    size_t token_quad = (size_t)(u / 4);
    size_t dim_in_16 = (size_t)(d % 16);
    size_t half = (size_t)((d / 16) % 2);
    size_t tok_in_quad = (size_t)(u % 4);
    within = (((dim_group * 4 + token_quad) * 16 + dim_in_16) * 2 + half) * 4 + tok_in_quad;
  }
  return tile + (size_t)sub * 16 * (size_t)D + within;
}

long oracle_pool_index(int is_v, long b, int h, int t, int d, int Hkv, int B, int D) {
  return (long)pool_index(is_v, b, h, t, d, Hkv, B, D);
}

/*
 * Byte index of (block b, kv head h, token slot t, dim d) in one layer's fp8 K or V pool. Same
 * tiles and 16-token sub-tiles as pool_index (one byte per element); inside a sub-tile, K is
 * ordered [d/64][(d/8)%4][token][(d/32)%2][d%8] and V [d/64][token/4][d%16][(d/16)%4][token%4].
 */
static size_t pool_index8(int is_v, long b, int h, int t, int d, int Hkv, int B, int D) {
  size_t tile = ((size_t)b * (size_t)Hkv + (size_t)h) * (size_t)B * (size_t)D;
  int sub = t / 16;
  int u = t % 16;
  size_t within;
  if (!is_v) {
    within = (size_t)(d / 64) * 1024 + (size_t)(16 * ((d / 8) % 4) + u) * 16 +
             (size_t)((d / 32) % 2) * 8 + (size_t)(d % 8);
  } else {
    within = (size_t)(d / 64) * 1024 + (size_t)((u / 4) * 16 + d % 16) * 16 +
             (size_t)((d / 16) % 4) * 4 + (size_t)(u % 4);
  }
  return tile + (size_t)sub * 16 * (size_t)D + within;
}

long oracle_pool_index8(int is_v, long b, int h, int t, int d, int Hkv, int B, int D) {
  return (long)pool_index8(is_v, b, h, t, d, Hkv, B, D);
}

/* oracle_gather for fp8 pools: values are e4m3_value(code) * scale. */
static int gather8(double* K_c, double* V_c, const uint8_t* k_pool, const uint8_t* v_pool,
                   double k_scale, double v_scale, const int32_t* table, int n, int g, int Hkv,
                   int D, int B, long num_blocks) {
  for (int t = 0; t < n; ++t) {
    long b = table[t / B];
    int slot = t % B;
    if (b < 0 || b >= num_blocks) return -1;
    for (int d = 0; d < D; ++d) {
      K_c[(size_t)t * D + d] = e4m3_value(k_pool[pool_index8(0, b, g, slot, d, Hkv, B, D)]) * k_scale;
      V_c[(size_t)t * D + d] = e4m3_value(v_pool[pool_index8(1, b, g, slot, d, Hkv, B, D)]) * v_scale;
    }
  }
  return 0;
}

/*
 * Reassemble the first n tokens of one sequence (block table row `table`) for kv head g into
 * contiguous K_c[n][D] and V_c[n][D]. Returns 0, or -1 if a table entry that is needed lies
 * outside [0, num_blocks).
 */
int oracle_gather(double* K_c, double* V_c, const uint16_t* k_pool, const uint16_t* v_pool,
                  int dtype, const int32_t* table, int n, int g, int Hkv, int D, int B,
                  long num_blocks) {
  for (int t = 0; t < n; ++t) {
    long b = table[t / B];
    int slot = t % B;
    if (b < 0 || b >= num_blocks) return -1;
    for (int d = 0; d < D; ++d) {
      K_c[(size_t)t * D + d] = elem_value(k_pool[pool_index(0, b, g, slot, d, Hkv, B, D)], dtype);
      V_c[(size_t)t * D + d] = elem_value(v_pool[pool_index(1, b, g, slot, d, Hkv, B, D)], dtype);
    }
  }
  return 0;
}

/* Dense single-query attention over contiguous rows, fp64: out[D]. */
static void dense_attention(double* out, const double* q, const double* K_c, const double* V_c,
                            int n, int D, double scale) {
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  if (n == 0) return;
  double* x = (double*)malloc(sizeof(double) * (size_t)n);
  double m = -INFINITY;
  for (int t = 0; t < n; ++t) {
    double dot = 0.0;
    for (int d = 0; d < D; ++d) dot += q[d] * K_c[(size_t)t * D + d];
    x[t] = scale * dot;
    if (x[t] > m) m = x[t];
  }
  double denom = 0.0;
  for (int t = 0; t < n; ++t) {
    double w = exp(x[t] - m);
    denom += w;
    for (int d = 0; d < D; ++d) out[d] += w * V_c[(size_t)t * D + d];
  }
  for (int d = 0; d < D; ++d) out[d] /= denom;
  free(x);
}

/*
 * Decode attention for a list of (sequence, query head) pairs (pairs[2*i], pairs[2*i+1]);
 * pairs == NULL means every pair in (s, h) order. out receives one row of D doubles per pair.
 * Returns 0, -1 on a bad table entry, -2 on bad arguments.
 */
int oracle_paged_decode(double* out, const uint16_t* q, const uint16_t* k_pool,
                        const uint16_t* v_pool, int dtype, const int32_t* block_tables,
                        const int32_t* context_lens, int num_seqs, int Hq, int Hkv, int D, int B,
                        long num_blocks, int max_blocks, float scale, const int32_t* pairs,
                        int npairs, int nthreads) {
  if (Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || B <= 0 || num_seqs < 0) return -2;
  int group = Hq / Hkv;
  long count = pairs ? (long)npairs : (long)num_seqs * Hq;
  int status = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
  for (long i = 0; i < count; ++i) {
    int s = pairs ? pairs[2 * i] : (int)(i / Hq);
    int h = pairs ? pairs[2 * i + 1] : (int)(i % Hq);
    double* row = out + (size_t)i * D;
    if (s < 0 || s >= num_seqs || h < 0 || h >= Hq) {
#pragma omp atomic write
      status = -2;
      continue;
    }
    int n = context_lens[s];
    if (n < 0 || n > max_blocks * B) {
#pragma omp atomic write
      status = -2;
      continue;
    }
    int g = h / group;
    double* qd = (double*)malloc(sizeof(double) * (size_t)D);
    double* K_c = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * D);
    double* V_c = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * D);
    for (int d = 0; d < D; ++d) qd[d] = elem_value(q[((size_t)s * Hq + h) * D + d], dtype);
    if (oracle_gather(K_c, V_c, k_pool, v_pool, dtype, block_tables + (size_t)s * max_blocks, n,
                      g, Hkv, D, B, num_blocks) != 0) {
#pragma omp atomic write
      status = -1;
    } else {
      dense_attention(row, qd, K_c, V_c, n, D, (double)scale);
    }
    free(qd);
    free(K_c);
    free(V_c);
  }
  return status;
}

/*
 * oracle_paged_decode over fp8 pools (scales k_scale, v_scale); q in bf16/fp16 (dtype).
 */
int oracle_paged_decode8(double* out, const uint16_t* q, const uint8_t* k_pool,
                         const uint8_t* v_pool, float k_scale, float v_scale, int dtype,
                         const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                         int Hq, int Hkv, int D, int B, long num_blocks, int max_blocks,
                         float scale, const int32_t* pairs, int npairs, int nthreads) {
  if (Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || B <= 0 || num_seqs < 0) return -2;
  int group = Hq / Hkv;
  long count = pairs ? (long)npairs : (long)num_seqs * Hq;
  int status = 0;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
#pragma omp parallel for schedule(dynamic, 1)
  for (long i = 0; i < count; ++i) {
    int s = pairs ? pairs[2 * i] : (int)(i / Hq);
    int h = pairs ? pairs[2 * i + 1] : (int)(i % Hq);
    double* row = out + (size_t)i * D;
    if (s < 0 || s >= num_seqs || h < 0 || h >= Hq) {
#pragma omp atomic write
      status = -2;
      continue;
    }
    int n = context_lens[s];
    if (n < 0 || n > max_blocks * B) {
#pragma omp atomic write
      status = -2;
      continue;
    }
    int g = h / group;
    double* qd = (double*)malloc(sizeof(double) * (size_t)D);
    double* K_c = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * D);
    double* V_c = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * D);
    for (int d = 0; d < D; ++d) qd[d] = elem_value(q[((size_t)s * Hq + h) * D + d], dtype);
    if (gather8(K_c, V_c, k_pool, v_pool, (double)k_scale, (double)v_scale,
                block_tables + (size_t)s * max_blocks, n, g, Hkv, D, B, num_blocks) != 0) {
#pragma omp atomic write
      status = -1;
    } else {
      dense_attention(row, qd, K_c, V_c, n, D, (double)scale);
    }
    free(qd);
    free(K_c);
    free(V_c);
  }
  return status;
}

/*
 * Host scatter into copies of one layer's fp8 pools: key/value are [T][Hkv][D] 16-bit words of
 * type dtype; the stored code is e4m3(fl32(x * fl32(1 / scale))). Returns 0, or -1 for a slot
 * beyond the pool.
 */
int oracle_reshape_and_cache8(uint8_t* k_pool, uint8_t* v_pool, const uint16_t* key,
                              const uint16_t* value, int dtype, float k_scale, float v_scale,
                              const int64_t* slot_mapping, int T, int Hkv, int D, int B,
                              long num_blocks) {
  volatile float one = 1.0f;  /* fp32 arithmetic, as stated above */
  float k_inv = one / k_scale;
  float v_inv = one / v_scale;
  for (int i = 0; i < T; ++i) {
    int64_t slot = slot_mapping[i];
    if (slot < 0) continue;
    if (slot >= (int64_t)num_blocks * B) return -1;
    long b = (long)(slot / B);
    int t = (int)(slot % B);
    for (int h = 0; h < Hkv; ++h) {
      for (int d = 0; d < D; ++d) {
        size_t src = ((size_t)i * Hkv + h) * D + d;
        float kx = (float)elem_value(key[src], dtype);
        float vx = (float)elem_value(value[src], dtype);
        float ky = kx * k_inv;
        float vy = vx * v_inv;
        k_pool[pool_index8(0, b, h, t, d, Hkv, B, D)] = e4m3_encode(ky);
        v_pool[pool_index8(1, b, h, t, d, Hkv, B, D)] = e4m3_encode(vy);
      }
    }
  }
  return 0;
}

/*
 * Host scatter of new tokens into a copy of one layer's pools. key/value are
 * [T][Hkv][D] 16-bit words; slots < 0 are skipped. Returns 0, or -1 if a slot lies at or
 * beyond num_blocks * B (nothing after it is written).
 */
int oracle_reshape_and_cache(uint16_t* k_pool, uint16_t* v_pool, const uint16_t* key,
                             const uint16_t* value, const int64_t* slot_mapping, int T, int Hkv,
                             int D, int B, long num_blocks) {
  for (int i = 0; i < T; ++i) {
    int64_t slot = slot_mapping[i];
    if (slot < 0) continue;
    if (slot >= (int64_t)num_blocks * B) return -1;
    long b = (long)(slot / B);
    int t = (int)(slot % B);
    for (int h = 0; h < Hkv; ++h) {
      for (int d = 0; d < D; ++d) {
        size_t src = ((size_t)i * Hkv + h) * D + d;
        k_pool[pool_index(0, b, h, t, d, Hkv, B, D)] = key[src];
        v_pool[pool_index(1, b, h, t, d, Hkv, B, D)] = value[src];
      }
    }
  }
  return 0;
}

/*
 * Pool indices of the dead slots of every sequence: slots t = n mod B .. B-1 of the block that
 * holds its last token, when that block is partly filled, for every kv head and dim (the slots a
 * decode must never read: "PagedAttention and KV Cache Management", section "How Block Paging
 * Operates During Generation": only the last block of a sequence is partly used). fp8 selects
 * pool_index8. Writes at most cap indices to out (out may be NULL) and returns how many there are.
 */
long oracle_dead_slot_indices(int is_v, int fp8, const int32_t* block_tables,
                              const int32_t* context_lens, int S, int max_blocks, int Hkv, int B,
                              int D, long* out, long cap) {
  long k = 0;
  for (int s = 0; s < S; ++s) {
    int n = context_lens[s];
    if (n <= 0 || n % B == 0) continue;
    long b = block_tables[(size_t)s * (size_t)max_blocks + (size_t)(n / B)];
    for (int t = n % B; t < B; ++t)
      for (int h = 0; h < Hkv; ++h)
        for (int d = 0; d < D; ++d) {
          if (out != NULL && k < cap)
            out[k] = (long)(fp8 ? pool_index8(is_v, b, h, t, d, Hkv, B, D)
                                : pool_index(is_v, b, h, t, d, Hkv, B, D));
          ++k;
        }
  }
  return k;
}

/*
 * Pool indices of whole token rows: for each slot of slots[0..n) that is >= 0 (slot = block * B
 * + t, the form reshape_and_cache takes), every kv head and dim, in that order. fp8 selects
 * pool_index8. Writes at most cap indices to out (out may be NULL); returns how many there are.
 */
long oracle_slot_indices(int is_v, int fp8, const int64_t* slots, int n, int Hkv, int B, int D,
                         long* out, long cap) {
  long k = 0;
  for (int i = 0; i < n; ++i) {
    if (slots[i] < 0) continue;
    long b = (long)(slots[i] / B);
    int t = (int)(slots[i] % B);
    for (int h = 0; h < Hkv; ++h)
      for (int d = 0; d < D; ++d) {
        if (out != NULL && k < cap)
          out[k] = (long)(fp8 ? pool_index8(is_v, b, h, t, d, Hkv, B, D)
                              : pool_index(is_v, b, h, t, d, Hkv, B, D));
        ++k;
      }
  }
  return k;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
