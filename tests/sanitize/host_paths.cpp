// Host-side test program for the sanitizer build of libpkdecode's host code
// (planner and C ABI), built with AddressSanitizer and UndefinedBehavior-
// Sanitizer on the CPU only: no kernel is launched and no GPU is needed.
//
//   host_paths partition   read partition cases from stdin, print each
//                          partition (the Python test compares them with the
//                          float64 oracle's rule, bit for bit)
//   host_paths abi         drive the C ABI's host paths: plans of random
//                          tables with explicit slot counts, their info and
//                          work lists, every argument check of plan, run,
//                          upload and merge_states that fails before any HIP
//                          call, and plans made from eight threads at once
//
// Exit status 0 when every check held; sanitizer reports abort the process.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <thread>
#include <vector>

#include "../../include/pkdecode.h"
#include "../../paged_kv_decode_plan_amd/csrc/planner.h"

namespace {

int g_failures = 0;

void check(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "CHECK FAILED: %s\n", what);
    ++g_failures;
  }
}

// Input: a case count, then per case
//   batch page_size units_per_item slots slots_per_cu balance min_chunk_pages
//   causal queries_per_item has_qo, indptr[batch+1], last_page_len[batch],
//   and qo_indptr[batch+1] when has_qo is 1.
// Output per case: "err <message>", or "ok <chunk_pages> <items> <partials>
// <splits>" followed by one line per item (8 columns), the merge index and
// the split requests.
int run_partitions() {
  int ncases = 0;
  if (std::scanf("%d", &ncases) != 1) return 2;
  for (int c = 0; c < ncases; ++c) {
    int B, P, units, slots, per_cu, balance, cmin, causal, qpi, has_qo;
    if (std::scanf("%d %d %d %d %d %d %d %d %d %d", &B, &P, &units, &slots, &per_cu, &balance,
                   &cmin, &causal, &qpi, &has_qo) != 10)
      return 2;
    // exact-size vectors, so that a read past the end is a sanitizer report
    std::vector<int32_t> indptr(size_t(B) + 1), last(static_cast<size_t>(B)), qo;
    for (auto& x : indptr) std::scanf("%d", &x);
    for (auto& x : last) std::scanf("%d", &x);
    if (has_qo) {
      qo.resize(size_t(B) + 1);
      for (auto& x : qo) std::scanf("%d", &x);
    }
    pkd::PartitionInput in;
    in.batch = B;
    in.indptr = indptr.data();
    in.last_page_len = last.data();
    in.qo_indptr = has_qo ? qo.data() : nullptr;
    in.queries_per_item = qpi;
    in.causal = causal != 0;
    in.page_size = P;
    in.units_per_item = units;
    in.slots = slots;
    in.slots_per_cu = per_cu;
    in.balance = balance;
    in.min_chunk_pages = cmin;
    pkd::Partition part;
    const std::string err = pkd::build_partition(in, &part);
    if (!err.empty()) {
      std::printf("err %s\n", err.c_str());
      continue;
    }
    std::printf("ok %d %zu %d %zu\n", part.chunk_pages, part.items.size(), part.num_partials,
                part.split_requests.size());
    for (const auto& w : part.items)
      std::printf("%d %d %d %d %d %d %d %d\n", w.request, w.page_begin, w.page_end, w.kv_len,
                  w.partial_slot, w.q_row, w.q_len, w.visible);
    for (const int32_t x : part.merge_indptr) std::printf("%d ", x);
    std::printf("\n");
    for (const int32_t x : part.split_requests) std::printf("%d ", x);
    std::printf("\n");
  }
  return 0;
}

struct Table {
  std::vector<int32_t> indptr, last;
};

Table random_table(std::mt19937& rng, int B, int P, int max_pages) {
  Table t;
  t.indptr.assign(1, 0);
  for (int r = 0; r < B; ++r) {
    t.indptr.push_back(t.indptr.back() + 1 + int(rng() % unsigned(max_pages)));
    t.last.push_back(1 + int(rng() % unsigned(P)));
  }
  return t;
}

pkd_plan_args plan_args(const Table& t, int P, int hq, int hkv, int kv_dtype, int slots) {
  pkd_plan_args a;
  std::memset(&a, 0, sizeof a);
  a.batch = int32_t(t.last.size());
  a.indptr = t.indptr.data();
  a.last_page_len = t.last.data();
  a.num_qo_heads = hq;
  a.num_kv_heads = hkv;
  a.head_dim = 128;
  a.page_size = P;
  a.q_dtype = PKD_DTYPE_BF16;
  a.kv_dtype = kv_dtype;
  a.out_dtype = PKD_DTYPE_BF16;
  a.slots = slots;
  return a;
}

// One plan of a random table: create, read info and work list, check that
// the work list covers every request's pages once, destroy.
bool plan_round_trip(std::mt19937& rng) {
  const int P = 1 << (rng() % 7);
  const int B = 1 + int(rng() % 200);
  Table t = random_table(rng, B, P, 1 + int(rng() % 400));
  static const int kv_forms[] = {PKD_DTYPE_BF16, PKD_DTYPE_E4M3, PKD_DTYPE_E2M1, PKD_DTYPE_I4};
  const int kv = kv_forms[rng() % 4];
  const int hkv = 1 << (rng() % 4);
  const int g = 1 << (rng() % 4);
  pkd_plan_args a = plan_args(t, P, hkv * g, hkv, kv, 1 + int(rng() % 4096));
  a.balance = int(rng() % 4);
  a.min_chunk_pages = int(rng() % 40);
  pkd_plan* p = nullptr;
  if (pkd_plan_create(&a, &p) != PKD_OK || !p) {
    std::fprintf(stderr, "plan failed: %s\n", pkd_last_error());
    return false;
  }
  pkd_plan_info info;
  bool ok = pkd_plan_get_info(p, &info) == PKD_OK;
  std::vector<int32_t> items(size_t(info.num_items) * PKD_ITEM_COLS);
  std::vector<int32_t> merge(size_t(B) + 1);
  std::vector<int32_t> split(static_cast<size_t>(info.num_split_requests));
  ok = ok && pkd_plan_get_worklist(p, items.data(), merge.data(), split.data()) == PKD_OK;
  std::vector<int64_t> covered(static_cast<size_t>(B), 0), tokens(static_cast<size_t>(B), 0);
  for (int32_t i = 0; ok && i < info.num_items; ++i) {
    const int32_t* row = &items[size_t(i) * PKD_ITEM_COLS];
    ok = row[0] >= 0 && row[0] < B && row[1] >= t.indptr[size_t(row[0])] &&
         row[2] <= t.indptr[size_t(row[0]) + 1] && row[2] > row[1];
    if (ok) {
      covered[size_t(row[0])] += row[2] - row[1];
      tokens[size_t(row[0])] += row[3];
    }
  }
  for (int r = 0; ok && r < B; ++r) {
    const int64_t n = t.indptr[size_t(r) + 1] - t.indptr[size_t(r)];
    ok = covered[size_t(r)] == n && tokens[size_t(r)] == (n - 1) * P + t.last[size_t(r)];
  }
  ok = ok && merge[0] == 0 && merge[size_t(B)] == info.num_partials;
  pkd_plan_destroy(p);
  return ok;
}

void check_argument_errors() {
  std::mt19937 rng(7);
  Table t = random_table(rng, 5, 16, 20);
  pkd_plan_args a = plan_args(t, 16, 32, 8, PKD_DTYPE_BF16, 256);
  pkd_plan* p = nullptr;

  check(pkd_plan_create(nullptr, &p) == PKD_ERR_INVALID_ARGUMENT, "null plan args");
  check(pkd_plan_create(&a, nullptr) == PKD_ERR_INVALID_ARGUMENT, "null plan out");
  {
    pkd_plan_args b = a;
    b.batch = 0;
    check(pkd_plan_create(&b, &p) == PKD_ERR_INVALID_ARGUMENT && p == nullptr, "empty batch");
  }
  {
    Table bad = t;
    bad.indptr[2] = bad.indptr[1];  // an empty request
    pkd_plan_args b = plan_args(bad, 16, 32, 8, PKD_DTYPE_BF16, 256);
    check(pkd_plan_create(&b, &p) == PKD_ERR_INVALID_ARGUMENT, "empty request");
    check(std::strstr(pkd_last_error(), "request") != nullptr, "error names the request");
  }
  {
    Table bad = t;
    bad.last[3] = 17;
    pkd_plan_args b = plan_args(bad, 16, 32, 8, PKD_DTYPE_BF16, 256);
    check(pkd_plan_create(&b, &p) == PKD_ERR_INVALID_ARGUMENT, "last_page_len above P");
  }
  {
    pkd_plan_args b = a;
    b.num_qo_heads = 30;
    check(pkd_plan_create(&b, &p) == PKD_ERR_INVALID_ARGUMENT, "Hq not a multiple of Hkv");
    b = a;
    b.head_dim = 96;
    check(pkd_plan_create(&b, &p) == PKD_ERR_UNSUPPORTED, "unsupported head_dim");
    b = a;
    b.page_size = 24;
    check(pkd_plan_create(&b, &p) == PKD_ERR_UNSUPPORTED, "page size not a power of two");
    b = a;
    b.kv_dtype = 99;
    check(pkd_plan_create(&b, &p) == PKD_ERR_UNSUPPORTED, "unknown kv dtype");
    b = a;
    b.sm_scale = -1.f;
    check(pkd_plan_create(&b, &p) == PKD_ERR_INVALID_ARGUMENT, "negative sm_scale");
    b = a;
    b.capacity_items = 4;
    check(pkd_plan_create(&b, &p) == PKD_ERR_INVALID_ARGUMENT, "partial capacities");
    b = a;
    b.kv_scale_per_token = 1;
    check(pkd_plan_create(&b, &p) == PKD_ERR_INVALID_ARGUMENT, "row-wise scales on bf16 KV");
    std::vector<int32_t> qo = {0, 1, 1, 2, 3, 4};  // request 1 without a query token
    b = a;
    b.qo_indptr = qo.data();
    check(pkd_plan_create(&b, &p) == PKD_ERR_INVALID_ARGUMENT, "request without queries");
  }

  check(pkd_plan_create(&a, &p) == PKD_OK && p, "valid plan");
  pkd_plan_info info;
  check(pkd_plan_get_info(p, nullptr) == PKD_ERR_INVALID_ARGUMENT, "null info");
  check(pkd_plan_get_info(p, &info) == PKD_OK, "info");
  check(pkd_plan_upload(p, nullptr, 1 << 20, nullptr) == PKD_ERR_INVALID_ARGUMENT, "null workspace");
  alignas(256) static unsigned char fake_ws[512];
  check(pkd_plan_upload(p, fake_ws, 1, nullptr) == PKD_ERR_WORKSPACE_TOO_SMALL,
        "upload into a small workspace");
  check(pkd_plan_upload(p, fake_ws + 16, 1 << 30, nullptr) == PKD_ERR_INVALID_ARGUMENT,
        "unaligned workspace");

  // run() checks its arguments before any HIP call; the pointers below are
  // never dereferenced on the host.
  alignas(16) static unsigned char fake[64];
  pkd_run_args r;
  std::memset(&r, 0, sizeof r);
  check(pkd_run(p, &r) == PKD_ERR_INVALID_ARGUMENT, "run without pointers");
  r.q = r.k = r.v = fake;
  r.indices = reinterpret_cast<const int32_t*>(fake);
  r.out = fake;
  r.workspace = fake_ws;
  r.workspace_bytes = sizeof fake_ws;
  check(pkd_run(p, &r) == PKD_ERR_PLAN_MISMATCH, "run on a workspace the plan was not uploaded to");
  check(pkd_run(nullptr, &r) == PKD_ERR_INVALID_ARGUMENT, "run without a plan");
  check(pkd_run_stages(p, &r, 0) == PKD_ERR_INVALID_ARGUMENT, "run with no stage");
  check(pkd_run_stages(p, &r, 4) == PKD_ERR_INVALID_ARGUMENT, "run with an unknown stage");
  pkd_plan_destroy(p);
  pkd_plan_destroy(nullptr);

  // merge_states: argument checks only (a valid call would launch)
  pkd_merge_states_args m;
  std::memset(&m, 0, sizeof m);
  check(pkd_merge_states(nullptr) == PKD_ERR_INVALID_ARGUMENT, "null merge args");
  m.rows = 4;
  m.num_heads = 2;
  m.head_dim = 6;
  check(pkd_merge_states(&m) == PKD_ERR_INVALID_ARGUMENT, "merge head_dim not a multiple of 4");
  m.head_dim = 128;
  m.in_dtype = PKD_DTYPE_E4M3;
  check(pkd_merge_states(&m) == PKD_ERR_UNSUPPORTED, "merge of fp8 rows");
  m.in_dtype = m.out_dtype = PKD_DTYPE_F32;
  check(pkd_merge_states(&m) == PKD_ERR_INVALID_ARGUMENT, "merge without pointers");
  m.rows = 0;
  check(pkd_merge_states(&m) == PKD_OK, "merge of no rows");

  int64_t bad = 0;
  check(pkd_check_page_ids(nullptr, 0, 10, nullptr, nullptr, nullptr) == PKD_ERR_INVALID_ARGUMENT,
        "page-id check without output");
  check(pkd_check_page_ids(nullptr, 5, 10, nullptr, &bad, nullptr) == PKD_ERR_INVALID_ARGUMENT,
        "page-id check without ids");
  check(pkd_version() > 0, "version");
}

int run_abi() {
  check_argument_errors();
  std::mt19937 rng(2026);
  for (int i = 0; i < 400; ++i) check(plan_round_trip(rng), "random plan round trip");
  // eight threads planning at once, each with its own generator
  std::vector<std::thread> threads;
  std::vector<int> thread_ok(8, 1);
  for (int t = 0; t < 8; ++t)
    threads.emplace_back([t, &thread_ok] {
      std::mt19937 r(100 + unsigned(t));
      for (int i = 0; i < 60; ++i) {
        if (!plan_round_trip(r)) thread_ok[size_t(t)] = 0;
        // a failing call between good ones: each thread's error message is its own
        pkd_plan_args a;
        std::memset(&a, 0, sizeof a);
        pkd_plan* p = nullptr;
        if (pkd_plan_create(&a, &p) != PKD_ERR_INVALID_ARGUMENT ||
            std::strstr(pkd_last_error(), "batch") == nullptr)
          thread_ok[size_t(t)] = 0;
      }
    });
  for (auto& th : threads) th.join();
  for (int t = 0; t < 8; ++t) check(thread_ok[size_t(t)] == 1, "threaded plans");
  std::printf("abi checks: %d failures\n", g_failures);
  return g_failures ? 1 : 0;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc < 2) {
    std::fprintf(stderr, "usage: %s partition|abi\n", argv[0]);
    return 2;
  }
  if (!std::strcmp(argv[1], "partition")) return run_partitions();
  if (!std::strcmp(argv[1], "abi")) return run_abi();
  return 2;
}
