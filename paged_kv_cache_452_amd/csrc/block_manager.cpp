// Host block manager of the C ABI (kv_block_manager_*): physical block bookkeeping for one pool.
//
// It decides, on the host, where each token's K and V go; the device work it implies is a
// reshape_and_cache of the new tokens into the returned slots, preceded by copy_blocks of the
// returned copy-on-write pairs. Rules ("PagedAttention and KV Cache Management" (blog.sejan.dev)):
//   * section "How Block Paging Operates During Generation": a prompt of n tokens gets
//     ceil(n / B) blocks (on-demand allocation); a generated token takes a new block only when it
//     starts a new logical block (boundary allocation);
//   * section "Advanced Memory Sharing: Prefix Caching & Copy-on-Write": fork shares every block
//     of the parent and raises its reference count; a token written into a block that other
//     sequences still reference first gets a private copy of that block;
//   * section "Hands-On Implementation: Building a PagedAttention Block Allocator in Python": free
//     blocks are handed out from the front of the free list and returned to its back, and running
//     out of blocks is an error.
// Swapping for preemption ("KV-Cache Management and PagedAttention", section "What paging unlocks
// downstream"; the same blog's section "Continuous Batching vs. Static Batching") keeps the same
// per-block accounting on a second, host-side set of blocks: a group of sequences moves together,
// each distinct block of the group's tables gets one block on the other side (front of that
// side's free list, in order of first appearance), so sharing inside the group survives; each
// table entry then drops its reference on the old block (blocks at zero go to the back of their
// free list in that same order). A swapped-out sequence cannot grow, fork or be decoded.
// Every operation either succeeds completely or changes nothing.

#include <stdint.h>
#include <stdlib.h>

#include <deque>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pagedkv.h"

struct pkv_block_manager {
  struct Seq {
    std::vector<int32_t> table;  // logical block -> physical block (host block when on_host)
    int64_t tokens = 0;
    bool on_host = false;        // swapped out
  };
  int num_blocks = 0;
  int block_size = 0;
  std::deque<int32_t> free_list;  // front: next block handed out
  std::vector<int32_t> refs;      // tables referencing each block
  std::deque<int32_t> host_free;  // the same for the host-side blocks of swapped-out sequences
  std::vector<int32_t> host_refs;
  std::unordered_map<int64_t, Seq> seqs;

  int32_t take() {
    const int32_t b = free_list.front();
    free_list.pop_front();
    refs[b] = 1;
    return b;
  }
  void drop(int32_t b) {
    if (--refs[b] == 0) free_list.push_back(b);
  }
};

namespace {

int64_t blocks_for(int64_t tokens, int block_size) { return (tokens + block_size - 1) / block_size; }

// Moves the group seq_ids to the host (to_host) or back to the device; see the rules at the top.
pkv_status move_group(pkv_block_manager* bm, const int64_t* seq_ids, int num_seqs, bool to_host,
                      int32_t* src_blocks, int32_t* dst_blocks, int max_pairs, int* num_pairs) {
  if (bm == nullptr || num_seqs < 0 || max_pairs < 0 || num_pairs == nullptr)
    return PKV_ERR_INVALID_ARG;
  *num_pairs = 0;
  if (num_seqs == 0) return PKV_OK;
  if (seq_ids == nullptr) return PKV_ERR_INVALID_ARG;
  std::unordered_set<int64_t> listed;
  std::vector<int32_t> order;  // distinct blocks in order of first appearance
  std::unordered_set<int32_t> seen;
  for (int i = 0; i < num_seqs; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end() || !listed.insert(seq_ids[i]).second) return PKV_ERR_INVALID_ARG;
    if (it->second.on_host == to_host) return PKV_ERR_INVALID_ARG;
    for (int32_t b : it->second.table) {
      if (seen.insert(b).second) order.push_back(b);
    }
  }
  std::vector<int32_t>& src_refs = to_host ? bm->refs : bm->host_refs;
  std::vector<int32_t>& dst_refs = to_host ? bm->host_refs : bm->refs;
  std::deque<int32_t>& src_free = to_host ? bm->free_list : bm->host_free;
  std::deque<int32_t>& dst_free = to_host ? bm->host_free : bm->free_list;
  if (order.size() > dst_free.size()) return PKV_ERR_NO_BLOCKS;
  if (order.size() > (size_t)max_pairs || (!order.empty() && (src_blocks == nullptr ||
                                                               dst_blocks == nullptr)))
    return PKV_ERR_INVALID_ARG;
  std::unordered_map<int32_t, int32_t> mapping;
  for (size_t k = 0; k < order.size(); ++k) {
    const int32_t nb = dst_free.front();
    dst_free.pop_front();
    dst_refs[nb] = 0;
    mapping.emplace(order[k], nb);
    src_blocks[k] = order[k];
    dst_blocks[k] = nb;
  }
  for (int i = 0; i < num_seqs; ++i) {
    pkv_block_manager::Seq& s = bm->seqs.find(seq_ids[i])->second;
    for (int32_t& b : s.table) {
      const int32_t nb = mapping.find(b)->second;
      ++dst_refs[nb];
      if (--src_refs[b] == 0) src_free.push_back(b);
      b = nb;
    }
    s.on_host = to_host;
  }
  *num_pairs = (int)order.size();
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status kv_block_manager_create(pkv_block_manager** out, int num_blocks, int num_host_blocks,
                                   int block_size) {
  if (out == nullptr) return PKV_ERR_INVALID_ARG;
  *out = nullptr;
  if (num_blocks <= 0 || num_host_blocks < 0 || block_size <= 0) return PKV_ERR_INVALID_ARG;
  pkv_block_manager* bm = new (std::nothrow) pkv_block_manager();
  if (bm == nullptr) return PKV_ERR_INVALID_ARG;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->refs.assign((size_t)num_blocks, 0);
  for (int32_t b = 0; b < num_blocks; ++b) bm->free_list.push_back(b);
  bm->host_refs.assign((size_t)num_host_blocks, 0);
  for (int32_t b = 0; b < num_host_blocks; ++b) bm->host_free.push_back(b);
  *out = bm;
  return PKV_OK;
}

void kv_block_manager_destroy(pkv_block_manager* bm) { delete bm; }

int kv_block_manager_num_free(const pkv_block_manager* bm) {
  return bm == nullptr ? -1 : (int)bm->free_list.size();
}

int kv_block_manager_num_free_host(const pkv_block_manager* bm) {
  return bm == nullptr ? -1 : (int)bm->host_free.size();
}

pkv_status kv_block_manager_allocate(pkv_block_manager* bm, int64_t seq_id, int64_t num_tokens) {
  if (bm == nullptr || num_tokens < 0) return PKV_ERR_INVALID_ARG;
  if (bm->seqs.count(seq_id)) return PKV_ERR_INVALID_ARG;
  const int64_t need = blocks_for(num_tokens, bm->block_size);
  if (need > (int64_t)bm->free_list.size()) return PKV_ERR_NO_BLOCKS;
  pkv_block_manager::Seq s;
  s.tokens = num_tokens;
  s.table.reserve((size_t)need);
  for (int64_t i = 0; i < need; ++i) s.table.push_back(bm->take());
  bm->seqs.emplace(seq_id, std::move(s));
  return PKV_OK;
}

pkv_status kv_block_manager_fork(pkv_block_manager* bm, int64_t src_seq_id, int64_t dst_seq_id) {
  if (bm == nullptr) return PKV_ERR_INVALID_ARG;
  auto it = bm->seqs.find(src_seq_id);
  if (it == bm->seqs.end() || bm->seqs.count(dst_seq_id)) return PKV_ERR_INVALID_ARG;
  if (it->second.on_host) return PKV_ERR_INVALID_ARG;
  pkv_block_manager::Seq copy = it->second;
  for (int32_t b : copy.table) ++bm->refs[b];
  bm->seqs.emplace(dst_seq_id, std::move(copy));
  return PKV_OK;
}

pkv_status kv_block_manager_append(pkv_block_manager* bm, const int64_t* seq_ids, int num_seqs,
                                   int64_t* slot_mapping, int32_t* copy_src, int32_t* copy_dst,
                                   int* num_copies) {
  if (bm == nullptr || num_seqs < 0 || num_copies == nullptr) return PKV_ERR_INVALID_ARG;
  *num_copies = 0;
  if (num_seqs == 0) return PKV_OK;
  if (seq_ids == nullptr || slot_mapping == nullptr || copy_src == nullptr || copy_dst == nullptr)
    return PKV_ERR_INVALID_ARG;
  const int B = bm->block_size;

  // Dry run: count the blocks the batch takes, following the same steps on shadow state (token
  // counts, whether the last block is already private, reference counts of touched blocks).
  {
    struct Shadow {
      int64_t tokens;
      bool last_private;  // last block taken or copied earlier in this batch
    };
    std::unordered_map<int64_t, Shadow> sh;
    std::unordered_map<int32_t, int32_t> refs;
    int64_t need = 0;
    for (int i = 0; i < num_seqs; ++i) {
      auto it = bm->seqs.find(seq_ids[i]);
      if (it == bm->seqs.end() || it->second.on_host) return PKV_ERR_INVALID_ARG;
      auto ins = sh.emplace(seq_ids[i], Shadow{it->second.tokens, false});
      Shadow& s = ins.first->second;
      if (s.tokens % B == 0) {
        ++need;
        s.last_private = true;
      } else if (!s.last_private) {
        const int32_t last = it->second.table[(size_t)(s.tokens / B)];
        auto r = refs.emplace(last, bm->refs[last]).first;
        if (r->second > 1) {
          ++need;
          --r->second;
        }
        s.last_private = true;  // either private already or now a private copy
      }
      ++s.tokens;
    }
    if (need > (int64_t)bm->free_list.size()) return PKV_ERR_NO_BLOCKS;
  }

  int n = 0;
  for (int i = 0; i < num_seqs; ++i) {
    pkv_block_manager::Seq& s = bm->seqs.find(seq_ids[i])->second;
    const int64_t pos = s.tokens;
    const size_t lb = (size_t)(pos / B);
    if (pos % B == 0) {
      s.table.push_back(bm->take());  // boundary: the token opens a new logical block
    } else {
      const int32_t last = s.table[lb];
      if (bm->refs[last] > 1) {  // copy-on-write: others still read this block
        const int32_t fresh = bm->take();
        --bm->refs[last];
        s.table[lb] = fresh;
        copy_src[n] = last;
        copy_dst[n] = fresh;
        ++n;
      }
    }
    s.tokens = pos + 1;
    slot_mapping[i] = (int64_t)s.table[lb] * B + pos % B;
  }
  *num_copies = n;
  return PKV_OK;
}

pkv_status kv_block_manager_release(pkv_block_manager* bm, int64_t seq_id) {
  if (bm == nullptr) return PKV_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return PKV_ERR_INVALID_ARG;
  if (it->second.on_host) {
    for (int32_t h : it->second.table) {
      if (--bm->host_refs[h] == 0) bm->host_free.push_back(h);
    }
  } else {
    for (int32_t b : it->second.table) bm->drop(b);
  }
  bm->seqs.erase(it);
  return PKV_OK;
}

pkv_status kv_block_manager_swap_out(pkv_block_manager* bm, const int64_t* seq_ids, int num_seqs,
                                     int32_t* device_blocks, int32_t* host_blocks, int max_pairs,
                                     int* num_pairs) {
  return move_group(bm, seq_ids, num_seqs, true, device_blocks, host_blocks, max_pairs,
                    num_pairs);
}

pkv_status kv_block_manager_swap_in(pkv_block_manager* bm, const int64_t* seq_ids, int num_seqs,
                                    int32_t* host_blocks, int32_t* device_blocks, int max_pairs,
                                    int* num_pairs) {
  return move_group(bm, seq_ids, num_seqs, false, host_blocks, device_blocks, max_pairs,
                    num_pairs);
}

pkv_status kv_block_manager_tables(const pkv_block_manager* bm, const int64_t* seq_ids,
                                   int num_seqs, int max_blocks_per_seq, int32_t* block_tables,
                                   int32_t* context_lens) {
  if (bm == nullptr || num_seqs < 0 || max_blocks_per_seq < 0) return PKV_ERR_INVALID_ARG;
  if (num_seqs == 0) return PKV_OK;
  if (seq_ids == nullptr || context_lens == nullptr ||
      (max_blocks_per_seq > 0 && block_tables == nullptr))
    return PKV_ERR_INVALID_ARG;
  for (int i = 0; i < num_seqs; ++i) {  // validate everything before writing anything
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end() || it->second.on_host) return PKV_ERR_INVALID_ARG;
    if ((int64_t)it->second.table.size() > max_blocks_per_seq || it->second.tokens > 2147483647)
      return PKV_ERR_INVALID_ARG;
  }
  for (int i = 0; i < num_seqs; ++i) {
    const pkv_block_manager::Seq& s = bm->seqs.find(seq_ids[i])->second;
    int32_t* row = block_tables + (size_t)i * max_blocks_per_seq;
    for (int j = 0; j < max_blocks_per_seq; ++j)
      row[j] = j < (int)s.table.size() ? s.table[(size_t)j] : -1;
    context_lens[i] = (int32_t)s.tokens;
  }
  return PKV_OK;
}

}  // extern "C"
