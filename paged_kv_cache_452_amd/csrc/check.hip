// paged_attention_check_inputs: a debug check of a decode step's index inputs, on the device.
//
// The decode and scatter kernels trust their indices: a used block-table entry outside the pool
// makes the decode read outside it, and a repeated slot makes reshape_and_cache's result depend
// on the order of its writes. The pages state these as properties of the bookkeeping -- a
// sequence's table names the pool blocks holding its tokens, and every token owns one slot
// ("PagedAttention and KV Cache Management" (blog.sejan.dev), sections "PagedAttention: OS
// Virtual Memory Architecture for GPUs" and "How Block Paging Operates During Generation"). This
// kernel counts violations without touching the pool, so it is safe to run on exactly the
// inputs it is meant to catch.

#include "pagedkv.h"

#include <hip/hip_runtime.h>

namespace {

constexpr int kCheckCounts = 4;  // bad table entries, bad lengths, repeated slots, slots past pool
constexpr int kCheckThreads = 256;  // threads of a check workgroup (the launch and the LDS tile)

struct CheckLaunch {
  const int32_t* block_tables;  // [num_seqs][max_blocks]
  const int32_t* context_lens;  // [num_seqs]
  const int64_t* slot_mapping;  // [num_tokens]; unused when num_tokens == 0
  unsigned* result;             // [kCheckCounts]
  int num_seqs;
  int max_blocks;
  int block_size;
  int num_blocks;
  int max_tokens;               // a context length above this is a violation
  int num_tokens;
  int64_t num_slots;            // num_blocks * block_size
};

__global__ __launch_bounds__(64) void zero_counts_kernel(unsigned* result) {
  if (threadIdx.x < kCheckCounts) result[threadIdx.x] = 0u;
}

// Sum of v over the wavefront, in lane 63 (every lane active).
__device__ __forceinline__ unsigned wave_sum(unsigned v) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) v += __shfl_xor(v, off);
  return v;
}

__global__ __launch_bounds__(kCheckThreads) void check_inputs_kernel(CheckLaunch a) {
  const long nthreads = (long)gridDim.x * blockDim.x;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  unsigned bad_entries = 0u, bad_lens = 0u, repeats = 0u, past = 0u;
  const long table_size = (long)a.num_seqs * a.max_blocks;
  const int row_tokens = a.max_blocks * a.block_size;
  // Context lengths (checked at a sequence's first entry) and the table entries they use: the
  // first ceil(n / block_size) of the row, with n clamped to the row as the decode clamps it.
  for (long e = gid; e < table_size; e += nthreads) {
    const int s = (int)(e / a.max_blocks);
    const int j = (int)(e - (long)s * a.max_blocks);
    const int n = a.context_lens[s];
    if (j == 0 && (n < 0 || n > a.max_tokens)) ++bad_lens;
    const int nc = n < 0 ? 0 : (n > row_tokens ? row_tokens : n);
    if (j < (nc + a.block_size - 1) / a.block_size) {
      const int b = a.block_tables[e];
      if (b < 0 || b >= a.num_blocks) ++bad_entries;
    }
  }
  // Sequences with no table row (max_blocks == 0) still have lengths to check.
  if (a.max_blocks == 0) {
    for (long s = gid; s < a.num_seqs; s += nthreads) {
      const int n = a.context_lens[s];
      if (n < 0 || n > a.max_tokens) ++bad_lens;
    }
  }
  // Slots: past the pool, and repeats (a non-negative slot equal to an earlier one). A workgroup
  // takes 256 consecutive tokens at a time (thread tid: token base + tid) and walks the slots
  // before them in tiles of 256 staged in LDS, each thread comparing its slot with the tile's
  // entries that precede it, 16 at a time (their LDS reads in flight together). The next tile's
  // entry is loaded into a register before the compares, so its latency hides behind them. The
  // loops are uniform over the workgroup (they depend on the base and num_tokens only), so every
  // thread reaches every barrier.
  constexpr int kCmp = 16;
  __shared__ int64_t s_tile[kCheckThreads];
  for (long base = (long)blockIdx.x * kCheckThreads; base < a.num_tokens;
       base += (long)gridDim.x * kCheckThreads) {
    const long i = base + threadIdx.x;
    const bool live = i < a.num_tokens;
    const int64_t si = live ? a.slot_mapping[i] : -1;
    if (live && si >= a.num_slots) ++past;
    bool found = false;
    const long kend = base + kCheckThreads < a.num_tokens ? base + kCheckThreads : a.num_tokens;
    int64_t next = (long)threadIdx.x < a.num_tokens ? a.slot_mapping[threadIdx.x] : -1;
    for (long k0 = 0; k0 < kend; k0 += kCheckThreads) {
      __syncthreads();  // the previous tile is no longer read
      s_tile[threadIdx.x] = next;
      __syncthreads();
      const long kn = k0 + kCheckThreads + threadIdx.x;
      next = (k0 + kCheckThreads < kend && kn < a.num_tokens) ? a.slot_mapping[kn] : -1;
      if (live && si >= 0 && !found) {
        const long before = i - k0;  // entries of this tile that precede token i
        const int n = before < kCheckThreads ? (int)before : kCheckThreads;
        for (int k1 = 0; k1 < n; k1 += kCmp) {
          int64_t e[kCmp];
#pragma unroll
          for (int u = 0; u < kCmp; ++u) e[u] = s_tile[k1 + u];
          bool hit = false;
#pragma unroll
          for (int u = 0; u < kCmp; ++u) hit |= (k1 + u < n) & (e[u] == si);
          if (hit) {
            found = true;
            break;
          }
        }
      }
    }
    if (found) ++repeats;
  }
  bad_entries = wave_sum(bad_entries);
  bad_lens = wave_sum(bad_lens);
  repeats = wave_sum(repeats);
  past = wave_sum(past);
  if ((threadIdx.x & 63) == 63) {
    if (bad_entries) atomicAdd(a.result + 0, bad_entries);
    if (bad_lens) atomicAdd(a.result + 1, bad_lens);
    if (repeats) atomicAdd(a.result + 2, repeats);
    if (past) atomicAdd(a.result + 3, past);
  }
}

}  // namespace

extern "C" pkv_status paged_attention_check_inputs(
    const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
    int max_blocks_per_seq, int max_context_len, int block_size, int num_blocks,
    const int64_t* slot_mapping, int num_tokens, int32_t* result, hipStream_t stream) {
  if (num_seqs < 0 || max_blocks_per_seq < 0 || max_context_len < 0 || block_size <= 0 ||
      num_blocks <= 0 || num_tokens < 0 || result == nullptr ||
      (num_seqs > 0 && (context_lens == nullptr ||
                        (max_blocks_per_seq > 0 && block_tables == nullptr))) ||
      (num_tokens > 0 && slot_mapping == nullptr))
    return PKV_ERR_INVALID_ARG;
  if ((long)max_blocks_per_seq * block_size > 2147483647L ||
      (long)num_seqs * max_blocks_per_seq > 2147483647L)
    return PKV_ERR_UNSUPPORTED;
  if (((uintptr_t)result & 3u) || ((uintptr_t)block_tables & 3u) ||
      ((uintptr_t)context_lens & 3u) || ((uintptr_t)slot_mapping & 7u))
    return PKV_ERR_ALIGNMENT;
  CheckLaunch a;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.slot_mapping = slot_mapping;
  a.result = (unsigned*)result;
  a.num_seqs = num_seqs;
  a.max_blocks = max_blocks_per_seq;
  a.block_size = block_size;
  a.num_blocks = num_blocks;
  const int row_tokens = max_blocks_per_seq * block_size;
  a.max_tokens = max_context_len < row_tokens ? max_context_len : row_tokens;
  a.num_tokens = num_tokens;
  a.num_slots = (int64_t)num_blocks * block_size;
  hipLaunchKernelGGL(zero_counts_kernel, dim3(1), dim3(64), 0, stream, a.result);
  const long entries = (long)num_seqs * (max_blocks_per_seq > 0 ? max_blocks_per_seq : 1);
  const long work = entries > num_tokens ? entries : (long)num_tokens;
  long blocks = (work + kCheckThreads - 1) / kCheckThreads;
  if (blocks < 1) blocks = 1;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(check_inputs_kernel, dim3((unsigned)blocks), dim3(kCheckThreads), 0, stream,
                     a);
  return hipGetLastError() == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}
