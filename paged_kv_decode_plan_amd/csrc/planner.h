// Host work partition for split-KV paged decode. Pure C++17: no HIP, so it
// can be built and tested on a machine without a GPU.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace pkd {

// One work item: a contiguous run of one request's pages.
struct WorkItem {
  int32_t request;
  int32_t page_begin;    // index into the page table (not a page id)
  int32_t page_end;      // exclusive
  int32_t kv_len;        // tokens covered
  int32_t partial_slot;  // -1: the item writes the output directly
};

struct PartitionInput {
  int32_t batch = 0;
  const int32_t* indptr = nullptr;         // [batch+1]
  const int32_t* last_page_len = nullptr;  // [batch]
  int32_t page_size = 0;
  int32_t units_per_item = 1;  // workgroups launched per item (one per KV head)
  int32_t slots = 1;           // workgroups resident on the device at once
  int32_t balance = 1;
  int32_t min_chunk_pages = 1;
};

struct Partition {
  int32_t chunk_pages = 0;
  std::vector<WorkItem> items;          // launch order
  std::vector<int32_t> merge_indptr;    // [batch+1]
  std::vector<int32_t> split_requests;  // ascending
  int32_t num_partials = 0;
  int64_t total_tokens = 0;
};

// Returns an empty string on success, else a description of what is wrong
// with the page table. The rule: a batch whose longest request is within 1/8
// of the mean (8 N B <= 9 S) and that gives at least half the resident slots
// in work units (2 B units >= slots) is not split (C = N); otherwise the chunk
// length is
//   C = min(N, max(min_chunk_pages, ceil(S * units / (slots * balance))))
// so that no work unit exceeds 1/balance of one slot's fair share. Request r
// becomes ceil(n_r / C) items; items are ordered by descending token count,
// ties by request then chunk index.
std::string build_partition(const PartitionInput& in, Partition* out);

}  // namespace pkd
