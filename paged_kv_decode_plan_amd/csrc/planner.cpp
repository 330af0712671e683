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
  if (in.units_per_item < 1 || in.slots < 1 || in.balance < 1 || in.min_chunk_pages < 1 ||
      in.queries_per_item < 1)
    return "units_per_item, slots, balance, min_chunk_pages and queries_per_item must be positive";
  if (in.indptr[0] != 0) return "indptr[0] must be 0";
  if (in.qo_indptr && in.qo_indptr[0] != 0) return "qo_indptr[0] must be 0";
  const int64_t Q = in.queries_per_item;

  int64_t total_pages = 0, max_pages = 0, total_tokens = 0;
  int64_t blocks = 0, block_pages = 0, max_q = 1;
  std::vector<int32_t> nq(B, 1);
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
    const int64_t L = (n - 1) * in.page_size + lp;
    if (in.qo_indptr) {
      const int64_t q = int64_t(in.qo_indptr[r + 1]) - in.qo_indptr[r];
      if (q < 1 || (in.causal && q > L)) {
        snprintf(msg, sizeof msg,
                 "request %d has %lld query tokens; it needs between 1 and its %lld KV tokens", r,
                 (long long)q, (long long)L);
        return msg;
      }
      nq[r] = int32_t(q);
      max_q = std::max(max_q, q);
    }
    total_pages += n;
    max_pages = std::max(max_pages, n);
    total_tokens += L;
    blocks += ceil_div(nq[r], Q);
    block_pages += n * ceil_div(nq[r], Q);
  }
  if (total_pages > INT32_MAX) return "page table longer than 2^31 entries";
  if (in.qo_indptr && int64_t(in.qo_indptr[B]) > INT32_MAX / 2) return "too many query rows";

  // A batch of near-equal requests is cut into k equal chunks per request,
  // k chosen to minimise the makespan of its work units over the compute
  // units: waves(k) = ceil(units * k / (CUs * balance)), each costing a chunk
  // (ceil(N / k) pages) plus a fixed 2 * min_chunk_pages for starting a
  // workgroup (and its share of the merge); ties keep the smaller k, and no chunk is
  // shorter than min_chunk_pages. (Several resident workgroups of one CU
  // share its bandwidth, so a CU, not a slot, is the machine here.)
  // Otherwise bound every work unit by 1/balance of a resident slot's fair
  // share (and by min_chunk_pages below).
  int64_t C;
  const bool near_equal = 8 * max_pages * blocks <= 9 * block_pages;
  if (near_equal) {
    const int64_t units = blocks * in.units_per_item;
    const int64_t resident =
        ceil_div(int64_t(in.slots), std::max<int64_t>(1, in.slots_per_cu)) * in.balance;
    const int64_t k_max = std::max<int64_t>(1, max_pages / in.min_chunk_pages);
    int64_t best_k = 1, best_cost = -1;
    for (int64_t k = 1; k <= k_max; ++k) {
      const int64_t cost =
          ceil_div(units * k, resident) * (ceil_div(max_pages, k) + 2 * int64_t(in.min_chunk_pages));
      if (best_cost < 0 || cost < best_cost) {
        best_cost = cost;
        best_k = k;
      }
    }
    C = ceil_div(max_pages, best_k);
  } else {
    const int64_t cap =
        ceil_div(block_pages * in.units_per_item, int64_t(in.slots) * in.balance);
    C = std::min<int64_t>(max_pages, std::max<int64_t>(in.min_chunk_pages, cap));
  }

  Partition p;
  p.chunk_pages = int32_t(C);
  p.total_tokens = total_tokens;
  p.query_rows = in.qo_indptr ? in.qo_indptr[B] : B;
  p.max_qo_len = int32_t(max_q);
  p.merge_indptr.assign(B + 1, 0);
  std::vector<int32_t> chunks(B);
  int64_t num_items = 0;
  for (int32_t r = 0; r < B; ++r) {
    const int64_t n = int64_t(in.indptr[r + 1]) - in.indptr[r];
    chunks[r] = int32_t(ceil_div(n, C));
    const int64_t rows = chunks[r] > 1 ? int64_t(chunks[r]) * nq[r] : 0;
    if (int64_t(p.merge_indptr[r]) + rows > INT32_MAX) return "too many partial states";
    p.merge_indptr[r + 1] = int32_t(p.merge_indptr[r] + rows);
    if (chunks[r] > 1) p.split_requests.push_back(r);
    num_items += int64_t(chunks[r]) * ceil_div(nq[r], Q);
  }
  if (num_items > INT32_MAX / 2) return "too many work items";
  p.num_partials = p.merge_indptr[B];

  struct Keyed {
    WorkItem w;
    int32_t chunk;
    int32_t block;
  };
  std::vector<Keyed> rows;
  rows.reserve(size_t(num_items));
  for (int32_t r = 0; r < B; ++r) {
    const int32_t end = in.indptr[r + 1];
    const int64_t L = int64_t(in.indptr[r + 1] - in.indptr[r] - 1) * in.page_size +
                      in.last_page_len[r];
    const int32_t q0 = in.qo_indptr ? in.qo_indptr[r] : r;
    const int32_t nblocks = int32_t(ceil_div(nq[r], Q));
    for (int32_t c = 0; c < chunks[r]; ++c) {
      WorkItem w;
      w.request = r;
      w.page_begin = int32_t(in.indptr[r] + int64_t(c) * C);
      w.page_end = int32_t(std::min<int64_t>(int64_t(w.page_begin) + C, end));
      w.kv_len = (w.page_end - w.page_begin) * in.page_size;
      if (w.page_end == end) w.kv_len -= in.page_size - in.last_page_len[r];
      for (int32_t b = 0; b < nblocks; ++b) {
        w.q_row = int32_t(q0 + b * Q);
        w.q_len = int32_t(std::min<int64_t>(Q, nq[r] - b * Q));
        // Tokens of this chunk the block's first token sees: everything up to its
        // own position L - q_r + b*Q, counted from the chunk's first token.
        w.visible = in.causal ? int32_t(std::min<int64_t>(
                                    w.kv_len, L - nq[r] + 1 + b * Q - int64_t(c) * C * in.page_size))
                              : w.kv_len;
        w.partial_slot =
            chunks[r] > 1 ? int32_t(p.merge_indptr[r] + int64_t(c) * nq[r] + b * Q) : -1;
        rows.push_back({w, c, b});
      }
    }
  }
  std::stable_sort(rows.begin(), rows.end(), [](const Keyed& a, const Keyed& b) {
    if (a.w.kv_len != b.w.kv_len) return a.w.kv_len > b.w.kv_len;
    if (a.w.request != b.w.request) return a.w.request < b.w.request;
    if (a.chunk != b.chunk) return a.chunk < b.chunk;
    return a.block < b.block;
  });
  p.items.reserve(rows.size());
  for (const auto& k : rows) p.items.push_back(k.w);
  *out = std::move(p);
  return std::string();
}

}  // namespace pkd
