// Host work partition for split-KV paged decode. Pure C++17: no HIP, so it
// can be built and tested on a machine without a GPU.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace pkd {

// One work item: a contiguous run of one request's pages, for a block of
// that request's new (query) tokens.
struct WorkItem {
  int32_t request;
  int32_t page_begin;    // index into the page table (not a page id)
  int32_t page_end;      // exclusive
  int32_t kv_len;        // tokens covered
  int32_t partial_slot;  // partial-state row of the block's first token; -1: writes the output
  int32_t q_row;         // q/out row of the block's first token
  int32_t q_len;         // tokens in the block (1 .. queries_per_item)
  int32_t visible;       // tokens of the item seen by the block's first token (token i
                         // sees min(kv_len, visible + i); <= 0: none)
};

struct PartitionInput {
  int32_t batch = 0;
  const int32_t* indptr = nullptr;         // [batch+1]
  const int32_t* last_page_len = nullptr;  // [batch]
  const int32_t* qo_indptr = nullptr;      // [batch+1] or NULL: one query token per request
  int32_t queries_per_item = 1;            // query tokens per work item
  bool causal = true;  // false: every q row sees all of its request's tokens
  int32_t page_size = 0;
  int32_t units_per_item = 1;  // workgroups launched per item (one per KV head)
  int32_t slots = 1;           // workgroups resident on the device at once
  int32_t slots_per_cu = 1;    // of which one compute unit holds (slots / this = CUs)
  int32_t balance = 1;
  int32_t min_chunk_pages = 1;
};

struct Partition {
  int32_t chunk_pages = 0;
  int32_t query_rows = 0;    // q/out rows (batch when one token per request)
  int32_t max_qo_len = 1;
  std::vector<WorkItem> items;          // launch order
  std::vector<int32_t> merge_indptr;    // [batch+1], in partial-state rows
  std::vector<int32_t> split_requests;  // ascending
  int32_t num_partials = 0;
  int64_t total_tokens = 0;
};

// Returns an empty string on success, else a description of what is wrong
// with the page table. The rule: a batch whose longest request is within 1/8
// of the mean (8 N B <= 9 S) is cut into k chunks per request, C = ceil(N/k),
// k in [1, max(1, N / min_chunk_pages)] minimising
//   ceil(B * units * k / (CUs * balance)) * (ceil(N / k) + 2 * min_chunk_pages)
// (waves of equal work units over the compute units, CUs = slots /
// slots_per_cu, each costing a chunk plus a workgroup's start), the smallest
// k on ties; otherwise the chunk length is
//   C = min(N, max(min_chunk_pages, ceil(S * units / (slots * balance))))
// so that no work unit exceeds 1/balance of one slot's fair share. Request r
// becomes ceil(n_r / C) items; items are ordered by descending token count,
// ties by request then chunk index.
//
// With several query tokens per request (qo_indptr), request r counts as
// ceil(q_r / queries_per_item) query blocks of n_r pages each: B and S above
// count blocks and their pages, every chunk is repeated per block, partial
// states are kept per query token (merge_indptr[r+1] - merge_indptr[r] =
// G_r * q_r when split), and ties go by request, chunk, then block. Without
// causality (the shared prefix of cascade attention) every row sees the whole
// item and q_r is not bounded by the request's token count.
std::string build_partition(const PartitionInput& in, Partition* out);

}  // namespace pkd
