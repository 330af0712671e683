// Host work partition for split-KV paged decode (see planner.h).
//
// FlashDecoding splits the KV axis into chunks that run as separate blocks
// and are merged afterwards; FlashInfer's plan balances that split so that a
// long request does not stall a batch of short ones ("FlashDecoding +
// FlashInfer — the decode-time attention story", §"FlashDecoding — the
// split-KV trick" and §"What FlashInfer is", item 3). The pages give no rule;
// the one implemented here bounds every work unit by a fraction of a resident
// workgroup slot's fair share of the whole batch.
#include "planner.h"

#include <algorithm>
#include <cstdio>

namespace pkd {

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

std::string build_partition(const PartitionInput& in, Partition* out) {
  char msg[256];
  const int32_t B = in.batch;
  if (B < 1) return "batch must be at least 1";
  if (!in.indptr || !in.last_page_len) return "indptr and last_page_len must not be NULL";
  if (in.page_size < 1) return "page_size must be positive";
  if (in.units_per_item < 1 || in.slots < 1 || in.balance < 1 || in.min_chunk_pages < 1)
    return "units_per_item, slots, balance and min_chunk_pages must be positive";
  if (in.indptr[0] != 0) return "indptr[0] must be 0";

  int64_t total_pages = 0, max_pages = 0, total_tokens = 0;
  for (int32_t r = 0; r < B; ++r) {
    const int64_t n = int64_t(in.indptr[r + 1]) - int64_t(in.indptr[r]);
    if (n < 1) {
      snprintf(msg, sizeof msg, "request %d has %lld pages; every request needs at least one", r,
               (long long)n);
      return msg;
    }
    const int32_t lp = in.last_page_len[r];
    if (lp < 1 || lp > in.page_size) {
      snprintf(msg, sizeof msg, "last_page_len[%d] = %d is outside [1, %d]", r, lp, in.page_size);
      return msg;
    }
    total_pages += n;
    max_pages = std::max(max_pages, n);
    total_tokens += (n - 1) * in.page_size + lp;
  }
  if (total_pages > INT32_MAX) return "page table longer than 2^31 entries";

  // A batch of near-equal requests that already yields at least half the
  // resident slots in work units is left whole: splitting it would only add
  // partial states and a merge. Otherwise bound every work unit by
  // 1/balance of a resident slot's fair share (and by min_chunk_pages below).
  int64_t C;
  const bool near_equal = 8 * max_pages * B <= 9 * total_pages;
  const bool enough_units = 2 * int64_t(B) * in.units_per_item >= in.slots;
  if (near_equal && enough_units) {
    C = max_pages;
  } else {
    const int64_t cap =
        ceil_div(total_pages * in.units_per_item, int64_t(in.slots) * in.balance);
    C = std::min<int64_t>(max_pages, std::max<int64_t>(in.min_chunk_pages, cap));
  }

  Partition p;
  p.chunk_pages = int32_t(C);
  p.total_tokens = total_tokens;
  p.merge_indptr.assign(B + 1, 0);
  std::vector<int32_t> chunks(B);
  for (int32_t r = 0; r < B; ++r) {
    const int64_t n = int64_t(in.indptr[r + 1]) - in.indptr[r];
    chunks[r] = int32_t(ceil_div(n, C));
    p.merge_indptr[r + 1] = p.merge_indptr[r] + (chunks[r] > 1 ? chunks[r] : 0);
    if (chunks[r] > 1) p.split_requests.push_back(r);
  }
  p.num_partials = p.merge_indptr[B];

  struct Keyed {
    WorkItem w;
    int32_t chunk;
  };
  std::vector<Keyed> rows;
  rows.reserve(size_t(p.merge_indptr[B]) + B);
  for (int32_t r = 0; r < B; ++r) {
    const int32_t end = in.indptr[r + 1];
    for (int32_t c = 0; c < chunks[r]; ++c) {
      WorkItem w;
      w.request = r;
      w.page_begin = int32_t(in.indptr[r] + int64_t(c) * C);
      w.page_end = int32_t(std::min<int64_t>(int64_t(w.page_begin) + C, end));
      w.kv_len = (w.page_end - w.page_begin) * in.page_size;
      if (w.page_end == end) w.kv_len -= in.page_size - in.last_page_len[r];
      w.partial_slot = chunks[r] > 1 ? p.merge_indptr[r] + c : -1;
      rows.push_back({w, c});
    }
  }
  std::stable_sort(rows.begin(), rows.end(), [](const Keyed& a, const Keyed& b) {
    if (a.w.kv_len != b.w.kv_len) return a.w.kv_len > b.w.kv_len;
    if (a.w.request != b.w.request) return a.w.request < b.w.request;
    return a.chunk < b.chunk;
  });
  p.items.reserve(rows.size());
  for (const auto& k : rows) p.items.push_back(k.w);
  *out = std::move(p);
  return std::string();
}

}  // namespace pkd
