// Paged-attention decode kernels for gfx950 (MI355X).
//
// One wavefront (64 lanes) owns one (sequence, kv head, group tile of <= 16 query heads,
// context partition). It walks the partition's logical blocks through the block table
// ("PagedAttention and KV Cache Management" (blog.sejan.dev), section "Under the Hood: The
// PagedAttention CUDA Kernel": physical_block_id = block_table[seq_id, logical_block_id]) and,
// per 16-token block:
//   * reads the K tile and the V tile straight from the pool: 64 lanes x 16 bytes per load
//     instruction, each instruction one contiguous 1 KiB range; the pool's tile order makes
//     every lane's 16 bytes a ready matrix-core operand, so nothing is staged or shuffled;
//   * scores S[token][head] = K_tile[16 x D] . Q^T[D x 16] with D/32 v_mfma_f32_16x16x32
//     (bf16 or f16) — all query heads of a GQA group share the one K read;
//   * keeps an online softmax with a lazily moved reference maximum: the reference m only moves
//     (and the running sum and output get rescaled) when a score exceeds it by more than 2^8,
//     so probabilities stay <= 256 and the common path needs no cross-lane traffic;
//   * accumulates O[head][dim] += P[head][token] . V_tile[token][dim] with v_mfma_f32_16x16x16,
//     P split into a 16-bit high part and a 16-bit residual so the product keeps fp32-level
//     precision of P;
// then either writes the normalised output (sequence fits one partition) or the partition's
// unnormalised (m, l, O) for the log-sum-exp merge kernel.
//
// Softmax identity used by the merge: with per-partition reference m_p, l_p = sum exp(x - m_p)
// and O_p = sum exp(x - m_p) v, the full result is
//   sum_p 2^(m_p - M) O_p / sum_p 2^(m_p - M) l_p   for any M (here M = max_p m_p),
// scores being kept in log2 units (x * scale * log2 e).

#include "pkv_internal.h"

namespace pkv {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// A score may exceed the reference maximum by this much (log2 units) before the reference moves.
constexpr float kLazyRescale = 8.0f;

// Tile buffers per wavefront (blocks in flight = kRing - 1), sized to stay within 256 VGPRs so
// two wavefronts fit on each SIMD.
template <int D>
constexpr int kRing = D == 128 ? 4 : 8;


template <bool BF16>
struct Elem;

template <>
struct Elem<true> {
  static __device__ __forceinline__ f32x4 qk(u32x4 k, u32x4 q, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k),
                                                   __builtin_bit_cast(bf16x8, q), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 pv(u32x2 p, u32x2 v, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, p),
                                                     __builtin_bit_cast(i16x4, v), c, 0, 0, 0);
  }
  // p = hi + lo (+ a residual below 2^-16 |p|), both parts 16-bit, packed in lane order.
  static __device__ __forceinline__ void split(const float p[4], u32x2& hi, u32x2& lo) {
    bf16x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[e] = (__bf16)p[e];
      l[e] = (__bf16)(p[e] - (float)h[e]);
    }
    hi = __builtin_bit_cast(u32x2, h);
    lo = __builtin_bit_cast(u32x2, l);
  }
  static __device__ __forceinline__ unsigned short store(float x) {
    return __builtin_bit_cast(unsigned short, (__bf16)x);
  }
};

template <>
struct Elem<false> {
  static __device__ __forceinline__ f32x4 qk(u32x4 k, u32x4 q, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, k),
                                                  __builtin_bit_cast(f16x8, q), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 pv(u32x2 p, u32x2 v, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, p),
                                                 __builtin_bit_cast(f16x4, v), c, 0, 0, 0);
  }
  static __device__ __forceinline__ void split(const float p[4], u32x2& hi, u32x2& lo) {
    f16x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[e] = (_Float16)p[e];
      l[e] = (_Float16)(p[e] - (float)h[e]);
    }
    hi = __builtin_bit_cast(u32x2, h);
    lo = __builtin_bit_cast(u32x2, l);
  }
  static __device__ __forceinline__ unsigned short store(float x) {
    return __builtin_bit_cast(unsigned short, (_Float16)x);
  }
};

__device__ __forceinline__ u32x4 load16(const char* p) { return *(const u32x4*)p; }

// K/V tiles are streamed: each is read once per launch, so the loads carry the non-temporal
// hint (measured on MI355X: random 4 KiB tile reads reach ~6.8 TB/s this way, ~6.05 TB/s with
// default-policy loads).
__device__ __forceinline__ u32x4 load16_stream(const char* p) {
  return __builtin_nontemporal_load((const u32x4*)p);
}

// Blocks of a partition [first, first + count) are split evenly over the partitions of a
// sequence: partition p of np covers blocks [p*nb/np, (p+1)*nb/np). Shared with the merge.
__device__ __forceinline__ int partitions_of(int n, int part_blocks, int max_parts) {
  const int nb = (n + kBlock - 1) / kBlock;
  // (clamped so that a context length above the promised maximum stays inside the workspace)
  return n > 0 ? min((nb + part_blocks - 1) / part_blocks, max_parts) : 1;
}

template <int D, bool BF16, int RING>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(2))) void
paged_decode_kernel(DecodeLaunch a) {
  using E = Elem<BF16>;
  constexpr int NQ = D / 32;   // 16-byte K loads (and QK matrix ops) per block
  constexpr int NV = D / 32;   // 16-byte V loads per block
  constexpr int NO = D / 16;   // 16-column output chunks
  constexpr size_t kTileBytes = (size_t)kBlock * D * 2;
  constexpr int kRow = D + 4;  // LDS row stride (floats) of the combine buffer

  __shared__ float sm_o[kWaves][kMaxGroupTile][kRow];
  __shared__ float sm_m[kWaves][kMaxGroupTile];
  __shared__ float sm_l[kWaves][kMaxGroupTile];

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int hl = lane & 15;    // query head within the tile (operand column)
  const int kg = lane >> 4;    // lane quarter: dims 8kg.. of each 32-dim chunk / tokens 4kg..

  int idx = blockIdx.x;
  const int ht = idx % a.head_tiles;
  idx /= a.head_tiles;
  const int g = idx % a.num_kv_heads;
  const int s = idx / a.num_kv_heads;
  const int part = blockIdx.y;

  const int n = a.context_lens[s];
  const int nparts = partitions_of(n, a.part_blocks, a.max_parts);
  if (part >= nparts) return;  // uniform over the workgroup
  const int nb_seq = (n + kBlock - 1) / kBlock;
  const int pb0 = (int)((long)part * nb_seq / nparts);        // partition's first block
  const int pb1 = (int)((long)(part + 1) * nb_seq / nparts);  // one past its last
  const int npb = pb1 - pb0;
  const int wb0 = pb0 + wave * npb / kWaves;                   // this wave's blocks
  const int nblk = pb0 + (wave + 1) * npb / kWaves - wb0;     // <= 64
  const int tok0 = wb0 * kBlock;
  const int tok1 = min(n, tok0 + nblk * kBlock);
  const int h0 = g * a.group + ht * kMaxGroupTile;
  const int nvalid = min(kMaxGroupTile, a.group - ht * kMaxGroupTile);

  // Block ids of this wave's blocks: lane i holds logical block wb0 + i.
  const int32_t* trow = a.block_tables + (size_t)s * a.max_blocks + wb0;
  const int bids = lane < nblk ? trow[lane] : 0;

  // Q^T operand: lane (hl, kg) holds q[h0 + hl][32c + 8kg .. +8] for each 32-dim chunk c.
  u32x4 qv[NQ];
  {
    const char* qrow = (const char*)a.q + ((size_t)s * a.num_q_heads + h0 + hl) * D * 2;
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
      qv[c] = hl < nvalid ? load16(qrow + (32 * c + 8 * kg) * 2) : u32x4{0u, 0u, 0u, 0u};
    }
  }

  const size_t blk_stride = (size_t)a.num_kv_heads * kTileBytes;
  const char* kbase = (const char*)a.k_pool + (size_t)g * kTileBytes + lane * 16;
  const char* vbase = (const char*)a.v_pool + (size_t)g * kTileBytes + lane * 16;

  float m_run = -INFINITY;  // reference maximum of head hl (log2 units)
  float l_run = 0.f;        // sum of p over this lane's tokens for head hl
  f32x4 o[NO];
#pragma unroll
  for (int i = 0; i < NO; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Ring of RING tile buffers: block j + RING - 1 is loading while block j is computed.
  u32x4 kr[RING][NQ], vr[RING][NV];
  auto issue = [&](int j, u32x4* kd, u32x4* vd) {
    const int b = __builtin_amdgcn_readlane(bids, j);
    const char* kp = kbase + (size_t)b * blk_stride;
    const char* vp = vbase + (size_t)b * blk_stride;
#pragma unroll
    for (int c = 0; c < NQ; ++c) kd[c] = load16_stream(kp + c * 1024);
#pragma unroll
    for (int c = 0; c < NV; ++c) vd[c] = load16_stream(vp + c * 1024);
  };

  auto process = [&](const u32x4* kc, u32x4* vc, int j) {
    // Scores: lane holds S[token 4kg + e][head hl], e = 0..3.
    f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NQ; ++c) sc = E::qk(kc[c], qv[c], sc);

    const int tb = tok0 + j * kBlock + 4 * kg;  // token of element e = 0
    float x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = (tb + e < tok1) ? sc[e] * a.scale_log2 : -INFINITY;
    const float lmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));

    if (__any(lmax > m_run + kLazyRescale)) {
      float gm = fmaxf(lmax, __shfl_xor(lmax, 16));
      gm = fmaxf(gm, __shfl_xor(gm, 32));
      const float m_new = fmaxf(m_run, gm);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ae = __shfl(alpha, 4 * kg + e);  // factor of output row (head 4kg + e)
#pragma unroll
        for (int i = 0; i < NO; ++i) o[i][e] *= ae;
      }
      m_run = m_new;
    }

    float p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] = __builtin_amdgcn_exp2f(x[e] - m_run);
    l_run += (p[0] + p[1]) + (p[2] + p[3]);
    u32x2 phi, plo;
    E::split(p, phi, plo);

    // Ragged last block: zero V of dead slots (they may hold anything, NaN included).
    if (tok0 + (j + 1) * kBlock > tok1) {
      const unsigned m01 = (tb + 0 < tok1 ? 0x0000FFFFu : 0u) | (tb + 1 < tok1 ? 0xFFFF0000u : 0u);
      const unsigned m23 = (tb + 2 < tok1 ? 0x0000FFFFu : 0u) | (tb + 3 < tok1 ? 0xFFFF0000u : 0u);
#pragma unroll
      for (int c = 0; c < NV; ++c) {
        vc[c].x &= m01;
        vc[c].y &= m23;
        vc[c].z &= m01;
        vc[c].w &= m23;
      }
    }

    // O[head][16i + col] += P[head][token] V[token][16i + col]
#pragma unroll
    for (int i = 0; i < NO; ++i) {
      const u32x4 w = vc[i / 2];
      const u32x2 vv = (i & 1) ? u32x2{w.z, w.w} : u32x2{w.x, w.y};
      o[i] = E::pv(phi, vv, o[i]);
      o[i] = E::pv(plo, vv, o[i]);
    }
  };

  // Prologue: blocks 0 .. RING-2 in flight.
#pragma unroll
  for (int u = 0; u < RING - 1; ++u) {
    if (u < nblk) issue(u, kr[u], vr[u]);
  }
  // Steady state: every iteration issues one block and computes one, with no conditions, so
  // the compiler can count outstanding loads exactly.
  const int steady = nblk >= RING - 1 ? (nblk - (RING - 1)) / RING * RING : 0;
  for (int j0 = 0; j0 < steady; j0 += RING) {
#pragma unroll
    for (int u = 0; u < RING; ++u) {
      issue(j0 + u + RING - 1, kr[(u + RING - 1) % RING], vr[(u + RING - 1) % RING]);
      process(kr[u], vr[u], j0 + u);
    }
  }
  // Tail: at most 2*RING - 2 blocks; block steady + u sits in slot u % RING.
#pragma unroll
  for (int u = 0; u < 2 * RING - 2; ++u) {
    const int j = steady + u;
    if (j < nblk) {
      if (j + RING - 1 < nblk) {
        issue(j + RING - 1, kr[(u + RING - 1) % RING], vr[(u + RING - 1) % RING]);
      }
      process(kr[u % RING], vr[u % RING], j);
    }
  }

  // Row sums of head hl over the four lane quarters.
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);

  // Combine the workgroup's waves: O_wg = sum_w 2^(m_w - M) O_w, L = sum_w 2^(m_w - M) l_w.
#pragma unroll
  for (int e = 0; e < 4; ++e) {
#pragma unroll
    for (int i = 0; i < NO; ++i) sm_o[wave][4 * kg + e][16 * i + hl] = o[i][e];
  }
  if (kg == 0) {
    sm_m[wave][hl] = m_run;
    sm_l[wave][hl] = l_tot;
  }
  __syncthreads();

  constexpr int kHeadsPerWave = kMaxGroupTile / kWaves;   // 4
  constexpr int kLanesPerHead = 64 / kHeadsPerWave;       // 16
  constexpr int kDims = D / kLanesPerHead;                // 8 (d128) or 4 (d64)
  const int head = wave * kHeadsPerWave + lane / kLanesPerHead;
  const int d0 = (lane % kLanesPerHead) * kDims;
  if (head >= nvalid) return;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm_m[w][head]);
  float L = 0.f;
  float acc[kDims];
#pragma unroll
  for (int i = 0; i < kDims; ++i) acc[i] = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const float mw = sm_m[w][head];
    const float c = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - M);  // empty wave -> 0
    L += c * sm_l[w][head];
#pragma unroll
    for (int i = 0; i < kDims; ++i) acc[i] += c * sm_o[w][head][d0 + i];
  }
  const size_t row = (size_t)s * a.num_q_heads + h0 + head;
  if (nparts == 1) {
    const float inv = L > 0.f ? 1.f / L : 0.f;   // n == 0 -> zeros
    unsigned short r[kDims];
#pragma unroll
    for (int i = 0; i < kDims; ++i) r[i] = E::store(acc[i] * inv);
    unsigned short* dst = (unsigned short*)a.out + row * D + d0;
    if constexpr (kDims == 8) {
      *(u32x4*)dst = u32x4{r[0] | (unsigned)r[1] << 16, r[2] | (unsigned)r[3] << 16,
                           r[4] | (unsigned)r[5] << 16, r[6] | (unsigned)r[7] << 16};
    } else {
      *(u32x2*)dst = u32x2{r[0] | (unsigned)r[1] << 16, r[2] | (unsigned)r[3] << 16};
    }
  } else {
    float* w = a.ws_o + (row * a.max_parts + part) * D + d0;
#pragma unroll
    for (int i = 0; i < kDims; ++i) w[i] = acc[i];
    if (lane % kLanesPerHead == 0) {
      float* ml = a.ws_ml + (row * a.max_parts + part) * 2;
      ml[0] = M;
      ml[1] = L;
    }
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Log-sum-exp merge of the partitions of one (sequence, query head).
template <int D, bool BF16>
__global__ __launch_bounds__(64) void merge_kernel(DecodeLaunch a) {
  using E = Elem<BF16>;
  constexpr int PER = D / 64;
  const int lane = threadIdx.x;
  const int s = blockIdx.x / a.num_q_heads;
  const int h = blockIdx.x % a.num_q_heads;
  const int n = a.context_lens[s];
  const int nparts = partitions_of(n, a.part_blocks, a.max_parts);
  if (nparts <= 1) return;
  const size_t base = ((size_t)s * a.num_q_heads + h) * a.max_parts;
  const float* ml = a.ws_ml + base * 2;

  float M = -INFINITY;
  for (int p = lane; p < nparts; p += 64) M = fmaxf(M, ml[2 * p]);
  M = wave_max(M);
  float L = 0.f;
  for (int p = lane; p < nparts; p += 64) L += __builtin_amdgcn_exp2f(ml[2 * p] - M) * ml[2 * p + 1];
  L = wave_sum(L);

  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  const float* op = a.ws_o + base * D + lane * PER;
  for (int p = 0; p < nparts; ++p) {
    const float w = __builtin_amdgcn_exp2f(ml[2 * p] - M);
#pragma unroll
    for (int i = 0; i < PER; ++i) acc[i] += w * op[(size_t)p * D + i];
  }
  const float inv = 1.f / L;
  unsigned short* out = (unsigned short*)a.out + ((size_t)s * a.num_q_heads + h) * D + lane * PER;
#pragma unroll
  for (int i = 0; i < PER; ++i) out[i] = E::store(acc[i] * inv);
}

template <int D, bool BF16>
hipError_t launch_typed(const DecodeLaunch& a, hipStream_t stream) {
  const dim3 grid((unsigned)(a.num_seqs * a.num_kv_heads * a.head_tiles), (unsigned)a.max_parts);
  hipLaunchKernelGGL((paged_decode_kernel<D, BF16, kRing<D>>), grid, dim3(64 * kWaves), 0, stream,
                     a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.max_parts <= 1) return err;
  hipLaunchKernelGGL((merge_kernel<D, BF16>), dim3((unsigned)(a.num_seqs * a.num_q_heads)),
                     dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeLaunch& a, int head_dim, bool bf16, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  if (head_dim == 128) return bf16 ? launch_typed<128, true>(a, stream) : launch_typed<128, false>(a, stream);
  return bf16 ? launch_typed<64, true>(a, stream) : launch_typed<64, false>(a, stream);
}

}  // namespace pkv
