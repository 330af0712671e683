// C-ABI surface of libpkdecode (declared in include/pkdecode.h).
//
// plan(): validate the page table, build the work partition on the host and
// lay out the device workspace; upload(): one asynchronous host-to-device copy
// of the work list; run(): the decode kernel and, when requests were split,
// the merge kernel. This mirrors the plan-once / run-per-layer wrapper of
// "FlashDecoding + FlashInfer — the decode-time attention story", §"The API
// you actually use (Python)".
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/pkdecode.h"
#include "launch.h"
#include "planner.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() { return PKD_OK; }

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// The workspace starts with a 256-byte block: the counts of a fixed-capacity
// plan at byte 0 and, at this offset, the two work counters of persistent
// decode launches (zero in every upload; the kernel leaves them at zero).
constexpr size_t kWorkCountersOffset = 128;

// 4-bit KV formats: two elements per byte.
bool nibbles(int dtype) { return dtype == PKD_DTYPE_E2M1 || dtype == PKD_DTYPE_I4; }

// Bytes of `elems` KV elements (4-bit formats: two per byte; odd counts are
// rejected by the callers' alignment checks before this matters).
int64_t kv_elems_bytes(int dtype, int64_t elems) {
  if (nibbles(dtype)) return elems / 2;
  return elems * (dtype == PKD_DTYPE_F32 ? 4 : (dtype == PKD_DTYPE_BF16 || dtype == PKD_DTYPE_F16) ? 2 : 1);
}

// Query / output element format as the kernels see it.
int kind_of(int dtype) {
  return dtype == PKD_DTYPE_BF16 ? pkd::kQBF16 : dtype == PKD_DTYPE_F16 ? pkd::kQF16 : pkd::kQF32;
}

// KV element format as the kernels see it (row-wise e4m3 scales are a form
// of their own).
int kv_form(int dtype, int per_token) {
  if (per_token) return pkd::kE4M3T;
  return dtype == PKD_DTYPE_F16    ? pkd::kF16
         : dtype == PKD_DTYPE_E2M1 ? pkd::kE2M1
         : dtype == PKD_DTYPE_I4   ? pkd::kI4
                                   : dtype;
}

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

// Pinned host staging blocks for plan uploads, shared by all plans of the
// process. A block goes back to the pool when its plan is destroyed and is
// handed out again only once the event recorded after its last copy has
// completed, so plan()/destroy() on the hot path allocate no pinned memory.
struct PinnedBlock {
  void* ptr = nullptr;
  size_t bytes = 0;
  hipEvent_t done = nullptr;  // recorded after the block's last copy
};

std::mutex g_pool_mu;
std::vector<PinnedBlock> g_pool;
constexpr size_t kPoolMax = 16;

int pinned_acquire(size_t need, PinnedBlock* out) {
  {
    std::lock_guard<std::mutex> lk(g_pool_mu);
    int best = -1;
    for (size_t i = 0; i < g_pool.size(); ++i) {
      if (g_pool[i].bytes < need) continue;
      if (hipEventQuery(g_pool[i].done) != hipSuccess) continue;  // still copying
      if (best < 0 || g_pool[i].bytes < g_pool[best].bytes) best = int(i);
    }
    if (best >= 0) {
      *out = g_pool[best];
      g_pool.erase(g_pool.begin() + best);
      return PKD_OK;
    }
  }
  size_t bytes = 64 * 1024;
  while (bytes < need) bytes *= 2;
  PinnedBlock b;
  b.bytes = bytes;
  hipError_t e = hipHostMalloc(&b.ptr, bytes, hipHostMallocDefault);
  if (e != hipSuccess) return fail(PKD_ERR_HIP, "hipHostMalloc(%zu): %s", bytes, hipGetErrorString(e));
  e = hipEventCreateWithFlags(&b.done, hipEventDisableTiming);
  if (e != hipSuccess) {
    (void)hipHostFree(b.ptr);
    return fail(PKD_ERR_HIP, "hipEventCreate: %s", hipGetErrorString(e));
  }
  *out = b;
  return PKD_OK;
}

void pinned_release(PinnedBlock b) {
  if (!b.ptr) return;
  std::lock_guard<std::mutex> lk(g_pool_mu);
  g_pool.push_back(b);
  while (g_pool.size() > kPoolMax) {
    // drop the smallest block whose copy has finished
    int victim = -1;
    for (size_t i = 0; i < g_pool.size(); ++i)
      if (hipEventQuery(g_pool[i].done) == hipSuccess &&
          (victim < 0 || g_pool[i].bytes < g_pool[victim].bytes))
        victim = int(i);
    if (victim < 0) break;
    (void)hipEventDestroy(g_pool[victim].done);
    (void)hipHostFree(g_pool[victim].ptr);
    g_pool.erase(g_pool.begin() + victim);
  }
}

// Resident workgroups per CU and CU count, per (device, kernel choice).
std::mutex g_slots_mu;
std::map<std::tuple<int, int, int, int, int, int, int, int, int>, std::pair<int, int>> g_slots;

// Decode workgroups per compute unit the library allows by default. One
// workgroup per CU (four wavefronts) is the fastest residency measured on
// MI355X for the one-token MFMA kernel on every bf16 and e4m3 workload (the
// eight KV heads of a work item are then read at the same time, and far
// fewer pages are open at once). The 4-bit forms (e2m1, int4) keep a SIMD
// 70-80 % busy widening codes and multiplying (VALU + MFMA busy counters),
// so more wavefronts per SIMD hide the loads one waits on: two workgroups
// per CU measured 8-9 % faster than one for both (and 8 % slower for e4m3);
// three were 4 % faster again for int4, the busiest, and 3 % slower for
// e2m1. Several new tokens per item carry more math per byte and keep the
// occupancy registers allow. 0: no cap.
int32_t default_wgs_cap(bool mfma, bool one_token, int kv_form) {
  if (!mfma || !one_token) return 0;
  return kv_form == pkd::kI4 ? 3 : kv_form == pkd::kE2M1 ? 2 : 1;
}

int device_slots(int32_t device, int32_t q_dtype, int32_t kv_dtype, int32_t head_dim,
                 int32_t group, int32_t rows, int32_t page_size, int32_t heads_per_wg,
                 int32_t wgs_cap, int32_t* wgs_per_cu, int32_t* num_cus) {
  const int q_kind = kind_of(q_dtype);
  if (!pkd::decode_supported(kv_dtype, head_dim, group, rows, q_kind, page_size))
    return fail(PKD_ERR_UNSUPPORTED,
                "no kernel for kv_dtype=%d head_dim=%d group=%d rows=%d q_dtype=%d", kv_dtype,
                head_dim, group, rows, q_dtype);
  const auto key = std::make_tuple(int(device), int(kv_dtype), int(head_dim), int(group),
                                   int(rows), q_kind, page_size >= 16 ? 16 : 1, int(wgs_cap),
                                   int(heads_per_wg));
  {
    std::lock_guard<std::mutex> lk(g_slots_mu);
    auto it = g_slots.find(key);
    if (it != g_slots.end()) {
      *wgs_per_cu = it->second.first;
      *num_cus = it->second.second;
      return ok();
    }
  }
  int prev = 0;
  hipError_t e = hipGetDevice(&prev);
  if (e != hipSuccess) return fail(PKD_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (prev != device && (e = hipSetDevice(device)) != hipSuccess)
    return fail(PKD_ERR_HIP, "hipSetDevice(%d): %s", device, hipGetErrorString(e));
  int cus = 0, wgs = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e == hipSuccess)
    e = pkd::decode_occupancy(kv_dtype, head_dim, group, rows, q_kind, page_size, heads_per_wg,
                              wgs_cap, &wgs);
  if (prev != device) (void)hipSetDevice(prev);
  if (e != hipSuccess) return fail(PKD_ERR_HIP, "device query: %s", hipGetErrorString(e));
  *wgs_per_cu = wgs;
  *num_cus = cus;
  std::lock_guard<std::mutex> lk(g_slots_mu);
  g_slots[key] = {wgs, cus};
  return ok();
}

}  // namespace

struct pkd_plan {
  pkd_plan_args args{};
  float sm_scale = 0.f;
  pkd::Partition part;
  pkd_plan_info info{};
  int rows = 0;  // query rows per work item and KV head (kernel choice)
  int heads_per_wg = 1;  // KV heads per decode workgroup (1, or 2: a pair)
  int kv_impl = 0;  // KV format as the kernels see it (pkd::kF32 .. kE4M3T)
  int wgs_cap = 0;  // decode workgroups per compute unit at most (0: no cap)
  bool fixed = false;    // fixed-capacity plan: grids from capacities, counts read on device
  int32_t launch_items = 0, launch_tasks = 0;
  // Device workspace layout (byte offsets).
  size_t off_items = 0, off_split = 0, off_blocks = 0, off_counters = 0, header_bytes = 0;
  int32_t num_blocks = 0;  // fused-merge records (split request, query block)
  bool fuse_ok = false;    // run() may fold the merge into the decode kernel
  size_t off_part_md = 0, off_part_o = 0;
  std::vector<unsigned char> header;  // host image of [items | merge tasks]
  PinnedBlock staging;                // from the process-wide pool, on first upload
  const void* uploaded_to = nullptr;
  int device = 0;
};

namespace {

// Argument checks shared by pkd_run_timed and pkd_run_static (everything but
// the workspace).
int check_run_args(const pkd_plan* p, const pkd_run_args* r, int32_t stages) {
  if (!p || !r) return fail(PKD_ERR_INVALID_ARGUMENT, "null argument");
  if (stages < 1 || stages > PKD_STAGE_ALL)
    return fail(PKD_ERR_INVALID_ARGUMENT, "stages must be a non-empty subset of PKD_STAGE_ALL");
  const pkd_plan_args& a = p->args;
  if (!r->q || !r->k || !r->v || !r->indices || !r->out)
    return fail(PKD_ERR_INVALID_ARGUMENT, "q, k, v, indices and out must not be NULL");
  if ((a.kv_dtype == PKD_DTYPE_E4M3 || nibbles(a.kv_dtype)) &&
      (!r->k_scale || !r->v_scale))
    return fail(PKD_ERR_INVALID_ARGUMENT, "e4m3, e2m1 and int4 KV need k_scale and v_scale");
  if ((a.kv_scale_per_token || nibbles(a.kv_dtype)) &&
      (reinterpret_cast<uintptr_t>(r->k_scale) % 16 || reinterpret_cast<uintptr_t>(r->v_scale) % 16))
    return fail(PKD_ERR_INVALID_ARGUMENT,
                "row-wise and per-channel scale arrays must be 16-byte aligned");
  const int vec_bytes = a.kv_dtype == PKD_DTYPE_E4M3 ? 8 : 16;
  const uintptr_t kp = reinterpret_cast<uintptr_t>(r->k), vp = reinterpret_cast<uintptr_t>(r->v);
  auto stride_ok = [&](int64_t st) {
    return (!nibbles(a.kv_dtype) || st % 2 == 0) &&
           kv_elems_bytes(a.kv_dtype, st) % vec_bytes == 0;
  };
  if (kp % vec_bytes || vp % vec_bytes || !stride_ok(r->page_stride) ||
      !stride_ok(r->token_stride) || !stride_ok(r->head_stride))
    return fail(PKD_ERR_INVALID_ARGUMENT,
                "k, v and the strides must be %d-byte aligned for 128-bit row loads", vec_bytes);
  if (reinterpret_cast<uintptr_t>(r->q) % 16)
    return fail(PKD_ERR_INVALID_ARGUMENT, "q must be 16-byte aligned");
  if (r->page_stride < 0 || r->token_stride < 0 || r->head_stride < 0)
    return fail(PKD_ERR_INVALID_ARGUMENT, "strides must be non-negative");
  // The decode kernels form a tile's address as 32-bit byte offsets within a
  // page on top of the page's 64-bit base.
  if (kv_elems_bytes(a.kv_dtype, r->page_stride) >= (int64_t(1) << 32))
    return fail(PKD_ERR_INVALID_ARGUMENT, "a page (page_stride) must span less than 4 GiB");
  if (!r->prior_out != !r->prior_lse)
    return fail(PKD_ERR_INVALID_ARGUMENT, "prior_out and prior_lse go together");
  if (r->prior_out && (reinterpret_cast<uintptr_t>(r->prior_out) % 16 ||
                       reinterpret_cast<uintptr_t>(r->prior_lse) % 4))
    return fail(PKD_ERR_INVALID_ARGUMENT, "prior_out must be 16-byte aligned");
  return PKD_OK;
}

// Enqueue the run's kernels with the plan's workspace image at `ws`.
int launch_run(const pkd_plan* p, const pkd_run_args* r, int32_t stages, char* ws,
               void* decode_start, void* decode_stop) {
  const pkd_plan_args& a = p->args;
  pkd::DecodeLaunch L;
  L.kv_dtype = p->kv_impl;
  L.head_dim = a.head_dim;
  L.group = a.num_qo_heads / a.num_kv_heads;
  L.rows = p->rows;
  L.wgs_cap = p->wgs_cap;
  L.heads_per_wg = p->heads_per_wg;
  L.num_items = p->launch_items;
  L.num_kv_heads = a.num_kv_heads;
  L.num_qo_heads = a.num_qo_heads;
  L.page_size_log2 = ilog2(a.page_size);
  L.sm_scale_log2 = float(double(p->sm_scale) * 1.4426950408889634);
  L.q_kind = kind_of(a.q_dtype);
  L.out_kind = kind_of(a.out_dtype);
  L.q = r->q;
  L.k = r->k;
  L.v = r->v;
  L.page_stride = r->page_stride;
  L.token_stride = r->token_stride;
  L.head_stride = r->head_stride;
  L.indices = r->indices;
  L.k_scale = r->k_scale;
  L.v_scale = r->v_scale;
  L.out = r->out;
  L.lse = r->lse;
  L.prior_out = r->prior_out;
  L.prior_lse = r->prior_lse;
  L.items = reinterpret_cast<const pkd::DeviceItem*>(ws + p->off_items);
  L.merge_tasks = reinterpret_cast<const pkd::MergeTask*>(ws + p->off_split);
  L.part_md = reinterpret_cast<float*>(ws + p->off_part_md);
  L.part_o = reinterpret_cast<float*>(ws + p->off_part_o);
  L.num_split = p->launch_tasks;
  L.counts = p->fixed ? reinterpret_cast<const int32_t*>(ws) : nullptr;
  L.work = reinterpret_cast<int32_t*>(ws + kWorkCountersOffset);
  L.block_merges = reinterpret_cast<const pkd::MergeTask*>(ws + p->off_blocks);
  L.counters = reinterpret_cast<int32_t*>(ws + p->off_counters);
  // A whole run of an exact plan whose split requests have at most
  // kFuseChunks chunks, over at most kFuseMaxWgs workgroups, folds the merge
  // into the decode kernel (one launch instead of two: what matters when the
  // batch is small). Longer folds run
  // faster in the separate merge kernel, which spreads them over many more
  // workgroups; fixed-capacity plans keep both launches so that one captured
  // graph fits every plan; the stages alone always keep them apart.
  L.fuse_merge = stages == PKD_STAGE_ALL && p->fuse_ok ? 1 : 0;
  hipStream_t s = static_cast<hipStream_t>(r->stream);
  hipError_t e;
  if (stages & PKD_STAGE_DECODE) {
    e = pkd::launch_decode(L, s, static_cast<hipEvent_t>(decode_start),
                           static_cast<hipEvent_t>(decode_stop));
    if (e != hipSuccess) return fail(PKD_ERR_HIP, "decode launch: %s", hipGetErrorString(e));
  }
  if ((stages & PKD_STAGE_MERGE) && !L.fuse_merge) {
    e = pkd::launch_merge(L, s);
    if (e != hipSuccess) return fail(PKD_ERR_HIP, "merge launch: %s", hipGetErrorString(e));
  }
  return ok();
}

}  // namespace

extern "C" {

const char* pkd_last_error(void) { return g_last_error.c_str(); }

int pkd_version(void) { return 300; }

int pkd_device_slots(int32_t device, int32_t q_dtype, int32_t kv_dtype, int32_t head_dim,
                     int32_t group, int32_t page_size, int32_t* wgs_per_cu, int32_t* num_cus) {
  if (!wgs_per_cu || !num_cus) return fail(PKD_ERR_INVALID_ARGUMENT, "null output pointer");
  const int form = kv_form(kv_dtype, 0);
  const bool mfma = pkd::decode_uses_mfma(form, head_dim, group, group, kind_of(q_dtype),
                                          page_size);
  // the kernel chosen for an even number of KV heads (head pairs where they apply)
  const int hp = pkd::decode_heads_per_wg(form, head_dim, group, group, kind_of(q_dtype),
                                          page_size, 2);
  return device_slots(device, q_dtype, form, head_dim, group, group, page_size, hp,
                      default_wgs_cap(mfma, true, form), wgs_per_cu, num_cus);
}

int pkd_plan_create(const pkd_plan_args* a, pkd_plan** out) {
  if (!a || !out) return fail(PKD_ERR_INVALID_ARGUMENT, "null argument");
  *out = nullptr;
  if (a->batch < 1) return fail(PKD_ERR_INVALID_ARGUMENT, "batch must be at least 1");
  if (!a->indptr || !a->last_page_len)
    return fail(PKD_ERR_INVALID_ARGUMENT, "indptr and last_page_len must not be NULL");
  if (a->num_qo_heads < 1 || a->num_kv_heads < 1 || a->num_qo_heads % a->num_kv_heads)
    return fail(PKD_ERR_INVALID_ARGUMENT,
                "num_qo_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                a->num_qo_heads, a->num_kv_heads);
  const int group = a->num_qo_heads / a->num_kv_heads;
  auto is_float = [](int d) {
    return d == PKD_DTYPE_F32 || d == PKD_DTYPE_BF16 || d == PKD_DTYPE_F16;
  };
  if (!is_float(a->q_dtype))
    return fail(PKD_ERR_UNSUPPORTED, "q_dtype %d not supported", a->q_dtype);
  if (!is_float(a->out_dtype))
    return fail(PKD_ERR_UNSUPPORTED, "out_dtype %d not supported", a->out_dtype);
  if (!is_float(a->kv_dtype) && a->kv_dtype != PKD_DTYPE_E4M3 && !nibbles(a->kv_dtype))
    return fail(PKD_ERR_UNSUPPORTED, "kv_dtype %d not supported", a->kv_dtype);
  if (a->kv_scale_per_token != 0 && a->kv_scale_per_token != 1)
    return fail(PKD_ERR_INVALID_ARGUMENT, "kv_scale_per_token must be 0 or 1");
  if (a->kv_scale_per_token && a->kv_dtype != PKD_DTYPE_E4M3)
    return fail(PKD_ERR_INVALID_ARGUMENT, "kv_scale_per_token applies to e4m3 KV only");
  // The kernels' view of the KV format: row-wise e4m3 scales are their own form.
  const int32_t kv_impl = kv_form(a->kv_dtype, a->kv_scale_per_token);
  const int q_kind = kind_of(a->q_dtype);
  if (!is_pow2(a->page_size) || a->page_size > 1024)
    return fail(PKD_ERR_UNSUPPORTED, "page_size %d is not a power of two in [1, 1024]",
                a->page_size);
  if (!pkd::decode_supported(kv_impl, a->head_dim, group, group,
                             q_kind, a->page_size))
    return fail(PKD_ERR_UNSUPPORTED,
                "no kernel for head_dim=%d group=%d kv_dtype=%d q_dtype=%d%s", a->head_dim, group,
                a->kv_dtype, a->q_dtype,
                a->kv_scale_per_token ? " with row-wise scales (needs bf16 q, head_dim 128)"
                : nibbles(a->kv_dtype) ? " (4-bit KV needs bf16 q and head_dim 128)"
                                                : "");
  // Several new tokens per request: a work item carries up to 16 / group (or
  // 32 / group, below) of one request's tokens, so that its group x tokens
  // rows fill one (two) groups of MFMA columns.
  int32_t max_q = 1;
  if (a->non_causal != 0 && a->non_causal != 1)
    return fail(PKD_ERR_INVALID_ARGUMENT, "non_causal must be 0 or 1");
  if (a->qo_indptr) {
    if (a->qo_indptr[0] != 0) return fail(PKD_ERR_INVALID_ARGUMENT, "qo_indptr[0] must be 0");
    for (int32_t r = 0; r < a->batch; ++r) {
      const int64_t q = int64_t(a->qo_indptr[r + 1]) - a->qo_indptr[r];
      if (q < 1)
        return fail(PKD_ERR_INVALID_ARGUMENT, "request %d has %lld query tokens", r, (long long)q);
      max_q = int32_t(std::min<int64_t>(std::max<int64_t>(max_q, q), INT32_MAX));
    }
  }
  // Fixed-capacity plans: everything the launch depends on comes from the
  // capacities (see the header), so the kernel choice uses capacity_qo_len.
  const int32_t caps[4] = {a->capacity_items, a->capacity_merge_tasks, a->capacity_partials,
                           a->capacity_qo_len};
  const bool fixed = caps[0] || caps[1] || caps[2] || caps[3];
  if (fixed && (caps[0] < 1 || caps[1] < 1 || caps[2] < 1 || caps[3] < 1))
    return fail(PKD_ERR_INVALID_ARGUMENT,
                "a fixed-capacity plan needs all four capacities positive (%d, %d, %d, %d)",
                caps[0], caps[1], caps[2], caps[3]);
  if (fixed && max_q > caps[3])
    return fail(PKD_ERR_INVALID_ARGUMENT, "a request has %d new tokens; capacity_qo_len is %d",
                max_q, caps[3]);
  const int32_t qo_shape = fixed ? caps[3] : max_q;
  // One column group (16 rows) per work item, or two (32 rows, sharing every
  // K/V load) when a request's new tokens need more than one group and the
  // KV form has the two-group kernel: fewer query blocks, fewer KV re-reads.
  int32_t queries_per_item = qo_shape > 1 ? std::max(1, 16 / group) : 1;
  if (qo_shape > 1 && qo_shape * group > 16 && group <= 16 &&
      pkd::decode_uses_mfma(kv_impl, a->head_dim, group, 32, q_kind, a->page_size))
    queries_per_item = 32 / group;
  const int32_t rows = group * std::min(queries_per_item, qo_shape);
  if (max_q > 1 && !pkd::decode_uses_mfma(kv_impl, a->head_dim, group, rows,
                                          q_kind, a->page_size))
    return fail(PKD_ERR_UNSUPPORTED,
                "several query tokens per request need head_dim 128 and bf16 q with bf16, e4m3, "
                "e2m1 or int4 KV, or fp16 q with fp16 KV "
                "(group %d, head_dim %d, kv_dtype %d, q_dtype %d)",
                group, a->head_dim, a->kv_dtype, a->q_dtype);
  if (a->slots < 0 || a->balance < 0 || a->min_chunk_pages < 0 || a->max_wgs_per_cu < 0)
    return fail(PKD_ERR_INVALID_ARGUMENT,
                "slots, balance, min_chunk_pages and max_wgs_per_cu must be >= 0");
  const bool mfma = pkd::decode_uses_mfma(kv_impl, a->head_dim, group, rows,
                                          q_kind, a->page_size);
  const int32_t wgs_cap =
      a->max_wgs_per_cu ? a->max_wgs_per_cu : default_wgs_cap(mfma, rows == group, kv_impl);
  // A workgroup per work item and KV head, or per pair of KV heads.
  const int32_t heads_per_wg = pkd::decode_heads_per_wg(kv_impl, a->head_dim, group, rows,
                                                        q_kind, a->page_size, a->num_kv_heads);
  if (!(a->sm_scale >= 0.f) || std::isinf(a->sm_scale))
    return fail(PKD_ERR_INVALID_ARGUMENT, "sm_scale must be finite and >= 0");

  int slots = a->slots;
  int slots_per_cu = 1;  // explicit slots are taken as one per compute unit
  if (slots == 0) {
    int32_t wgs = 0, cus = 0;
    int rc = device_slots(a->device, a->q_dtype, kv_impl, a->head_dim, group, rows,
                          a->page_size, heads_per_wg, wgs_cap, &wgs, &cus);
    if (rc != PKD_OK) return rc;
    slots = wgs * cus;
    slots_per_cu = std::max(1, int(wgs));
    if (slots < 1) return fail(PKD_ERR_HIP, "device reports no resident workgroups");
  }
  pkd::PartitionInput pin;
  pin.batch = a->batch;
  pin.indptr = a->indptr;
  pin.last_page_len = a->last_page_len;
  pin.qo_indptr = max_q > 1 ? a->qo_indptr : nullptr;
  pin.queries_per_item = queries_per_item;
  pin.causal = a->non_causal == 0;
  pin.page_size = a->page_size;
  pin.units_per_item = a->num_kv_heads / heads_per_wg;
  pin.slots = slots;
  pin.slots_per_cu = slots_per_cu;
  pin.balance = a->balance ? a->balance : 1;
  // Default shortest chunk: 64 tokens. It binds only for a batch too small to
  // give every slot a share of that size, where the step is latency-bound and
  // more, shorter chunks finish sooner (the single-sequence workload: 21.0 us
  // per step with 256-token chunks, 12.6 us with 64).
  pin.min_chunk_pages = a->min_chunk_pages ? a->min_chunk_pages : (64 + a->page_size - 1) / a->page_size;

  pkd_plan* p = new (std::nothrow) pkd_plan();
  if (!p) return fail(PKD_ERR_INVALID_ARGUMENT, "out of host memory");
  std::string err = pkd::build_partition(pin, &p->part);
  if (!err.empty()) {
    delete p;
    return fail(PKD_ERR_INVALID_ARGUMENT, "%s", err.c_str());
  }
  p->args = *a;
  p->args.indptr = nullptr;
  p->args.last_page_len = nullptr;
  p->args.qo_indptr = nullptr;
  p->rows = rows;
  p->kv_impl = kv_impl;
  p->wgs_cap = wgs_cap;
  p->heads_per_wg = heads_per_wg;
  p->device = a->device;
  p->sm_scale = a->sm_scale > 0.f ? a->sm_scale : 1.0f / std::sqrt(float(a->head_dim));

  const auto& part = p->part;
  const size_t n_items = part.items.size();
  const size_t n_split = part.split_requests.size();
  // One merge task per q row of a split request.
  std::vector<pkd::MergeTask> tasks;
  for (const int32_t r : part.split_requests) {
    const int32_t q0 = max_q > 1 ? a->qo_indptr[r] : r;
    const int32_t nq = max_q > 1 ? a->qo_indptr[r + 1] - a->qo_indptr[r] : 1;
    const int32_t chunks = (part.merge_indptr[r + 1] - part.merge_indptr[r]) / nq;
    for (int32_t i = 0; i < nq; ++i) tasks.push_back({q0 + i, part.merge_indptr[r] + i, chunks, nq});
  }
  const size_t n_tasks = tasks.size();
  // One fused-merge record per (split request, query block); the item's
  // record index is found from its first q row.
  std::vector<pkd::MergeTask> blocks;
  std::map<int32_t, int32_t> block_of_row;
  for (const int32_t r : part.split_requests) {
    const int32_t q0 = max_q > 1 ? a->qo_indptr[r] : r;
    const int32_t nq = max_q > 1 ? a->qo_indptr[r + 1] - a->qo_indptr[r] : 1;
    const int32_t chunks = (part.merge_indptr[r + 1] - part.merge_indptr[r]) / nq;
    for (int32_t b = 0; b * queries_per_item < nq; ++b) {
      block_of_row[q0 + b * queries_per_item] = int32_t(blocks.size());
      blocks.push_back({q0 + b * queries_per_item, part.merge_indptr[r] + b * queries_per_item,
                        chunks, nq});
    }
  }
  const size_t n_blocks = blocks.size();
  constexpr int32_t kFuseChunks = 16;
  int32_t max_chunks = 0;
  for (const auto& b : blocks) max_chunks = std::max(max_chunks, b.count);
  if (fixed && (n_items > size_t(caps[0]) || n_tasks > size_t(caps[1]) ||
                size_t(part.num_partials) > size_t(caps[2]))) {
    const size_t np = size_t(part.num_partials);
    delete p;
    return fail(PKD_ERR_INVALID_ARGUMENT,
                "the plan needs %zu work items, %zu merge tasks and %zu partial rows; the "
                "capacities are %d, %d and %d",
                n_items, n_tasks, np, caps[0], caps[1], caps[2]);
  }
  // Workspace: [counts and work counters (256 B) | items | merge tasks | fused-merge records |
  // fused-merge counters | partial (m, d) | partial o], sized by the plan
  // itself or, for a fixed-capacity plan, by its capacities (records never
  // outnumber merge tasks). The uploaded header runs through the counters,
  // so every upload starts them at zero; the kernel leaves them at zero.
  const size_t lay_items = fixed ? size_t(caps[0]) : n_items;
  const size_t lay_tasks = fixed ? size_t(caps[1]) : std::max<size_t>(n_tasks, 1);
  const size_t lay_parts = fixed ? size_t(caps[2]) : size_t(part.num_partials);
  p->fixed = fixed;
  p->launch_items = int32_t(lay_items);
  p->launch_tasks = fixed ? caps[1] : int32_t(n_tasks);
  p->num_blocks = int32_t(n_blocks);
  // Folding costs every split workgroup a device-scope release (and the last
  // one an acquire), which on MI355X write back and invalidate its XCD's L2:
  // cheaper than the merge launch for a few workgroups (the single-sequence
  // step, 512 tokens in eight chunks over four KV heads: 12.7 -> 11.9 us),
  // dearer for hundreds (64 requests split in two over eight KV heads: 94.0
  // -> 99.4 us; 32-chunk requests: 166.6 -> 177.2 us).
  constexpr size_t kFuseMaxWgs = 64;
  size_t split_wgs = 0;
  for (const auto& it : part.items)
    if (it.partial_slot >= 0) split_wgs += size_t(pin.units_per_item);
  p->fuse_ok = !fixed && max_chunks <= kFuseChunks && split_wgs <= kFuseMaxWgs;
  p->off_items = 256;
  p->off_split = align256(p->off_items + lay_items * sizeof(pkd::DeviceItem));
  p->off_blocks = align256(p->off_split + lay_tasks * sizeof(pkd::MergeTask));
  p->off_counters = align256(p->off_blocks + lay_tasks * sizeof(pkd::MergeTask));
  const size_t end_counters =
      align256(p->off_counters + lay_tasks * size_t(a->num_kv_heads) * sizeof(int32_t));
  p->header_bytes = p->off_counters + std::max<size_t>(n_blocks, 1) *
                                          size_t(a->num_kv_heads) * sizeof(int32_t);
  p->off_part_md = end_counters;
  const size_t prows = lay_parts * size_t(a->num_qo_heads);
  p->off_part_o = align256(p->off_part_md + prows * 2 * sizeof(float));
  const size_t ws = align256(p->off_part_o + prows * size_t(a->head_dim) * sizeof(float));

  p->header.assign(p->header_bytes, 0);
  reinterpret_cast<int32_t*>(p->header.data())[0] = int32_t(n_items);
  reinterpret_cast<int32_t*>(p->header.data())[1] = int32_t(n_tasks);
  auto* di = reinterpret_cast<pkd::DeviceItem*>(p->header.data() + p->off_items);
  for (size_t i = 0; i < n_items; ++i) {
    const auto& w = part.items[i];
    // The kernel reads only the tokens some row of the block sees.
    const int64_t seen = std::max<int64_t>(
        0, std::min<int64_t>(w.kv_len, int64_t(w.visible) + w.q_len - 1));
    const int32_t blk = w.partial_slot >= 0 ? block_of_row.at(w.q_row) : -1;
    di[i] = {w.page_begin, int32_t(seen), w.partial_slot, w.q_row, w.q_len, w.visible, blk, 0};
  }
  if (n_tasks)
    std::memcpy(p->header.data() + p->off_split, tasks.data(), n_tasks * sizeof(pkd::MergeTask));
  if (n_blocks)
    std::memcpy(p->header.data() + p->off_blocks, blocks.data(),
                n_blocks * sizeof(pkd::MergeTask));

  pkd_plan_info& inf = p->info;
  inf.batch = a->batch;
  inf.chunk_pages = part.chunk_pages;
  inf.num_items = int32_t(n_items);
  inf.num_partials = part.num_partials;
  inf.num_split_requests = int32_t(n_split);
  inf.slots = pin.slots;
  inf.balance = pin.balance;
  inf.min_chunk_pages = pin.min_chunk_pages;
  inf.total_kv_tokens = part.total_tokens;
  inf.workspace_bytes = ws;
  inf.query_rows = part.query_rows;
  inf.queries_per_item = queries_per_item;
  inf.max_qo_len = max_q;
  inf.num_merge_tasks = int32_t(n_tasks);
  inf.units_per_item = pin.units_per_item;
  inf.slots_per_cu = pin.slots_per_cu;
  inf.merge_folded = p->fuse_ok && n_split > 0 ? 1 : 0;
  *out = p;
  return ok();
}

int pkd_plan_get_info(const pkd_plan* p, pkd_plan_info* info) {
  if (!p || !info) return fail(PKD_ERR_INVALID_ARGUMENT, "null argument");
  *info = p->info;
  return ok();
}

int pkd_plan_get_worklist(const pkd_plan* p, int32_t* items_out, int32_t* merge_indptr_out,
                          int32_t* split_requests_out) {
  if (!p) return fail(PKD_ERR_INVALID_ARGUMENT, "null plan");
  if (items_out) {
    for (size_t i = 0; i < p->part.items.size(); ++i) {
      const auto& w = p->part.items[i];
      int32_t* row = items_out + i * PKD_ITEM_COLS;
      row[0] = w.request;
      row[1] = w.page_begin;
      row[2] = w.page_end;
      row[3] = w.kv_len;
      row[4] = w.partial_slot;
      row[5] = w.q_row;
      row[6] = w.q_len;
      row[7] = w.visible;
    }
  }
  if (merge_indptr_out)
    std::memcpy(merge_indptr_out, p->part.merge_indptr.data(), p->part.merge_indptr.size() * 4);
  if (split_requests_out && !p->part.split_requests.empty())
    std::memcpy(split_requests_out, p->part.split_requests.data(),
                p->part.split_requests.size() * 4);
  return ok();
}

int pkd_plan_upload(pkd_plan* p, void* workspace, size_t workspace_bytes, void* stream) {
  if (!p || !workspace) return fail(PKD_ERR_INVALID_ARGUMENT, "null plan or workspace");
  if (workspace_bytes < p->info.workspace_bytes)
    return fail(PKD_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, the plan needs %zu",
                workspace_bytes, p->info.workspace_bytes);
  if (reinterpret_cast<uintptr_t>(workspace) % 256)
    return fail(PKD_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
  hipError_t e;
  if (!p->staging.ptr) {
    const int rc = pinned_acquire(p->header_bytes, &p->staging);
    if (rc != PKD_OK) return rc;
  } else if ((e = hipEventSynchronize(p->staging.done)) != hipSuccess) {
    return fail(PKD_ERR_HIP, "waiting for the previous upload: %s", hipGetErrorString(e));
  }
  std::memcpy(p->staging.ptr, p->header.data(), p->header_bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((e = hipMemcpyAsync(workspace, p->staging.ptr, p->header_bytes, hipMemcpyHostToDevice, s)) !=
      hipSuccess)
    return fail(PKD_ERR_HIP, "hipMemcpyAsync: %s", hipGetErrorString(e));
  if ((e = hipEventRecord(p->staging.done, s)) != hipSuccess)
    return fail(PKD_ERR_HIP, "hipEventRecord: %s", hipGetErrorString(e));
  p->uploaded_to = workspace;
  return ok();
}

int pkd_run(const pkd_plan* p, const pkd_run_args* r) { return pkd_run_stages(p, r, PKD_STAGE_ALL); }

int pkd_run_stages(const pkd_plan* p, const pkd_run_args* r, int32_t stages) {
  return pkd_run_timed(p, r, stages, nullptr, nullptr);
}

int pkd_run_timed(const pkd_plan* p, const pkd_run_args* r, int32_t stages, void* decode_start,
                  void* decode_stop) {
  if (int rc = check_run_args(p, r, stages); rc != PKD_OK) return rc;
  if (!r->workspace) return fail(PKD_ERR_INVALID_ARGUMENT, "workspace must not be NULL");
  if (r->workspace != p->uploaded_to)
    return fail(PKD_ERR_PLAN_MISMATCH, "workspace differs from the one the plan was uploaded to");
  if (r->workspace_bytes < p->info.workspace_bytes)
    return fail(PKD_ERR_WORKSPACE_TOO_SMALL, "workspace has %zu bytes, the plan needs %zu",
                r->workspace_bytes, p->info.workspace_bytes);
  return launch_run(p, r, stages, static_cast<char*>(r->workspace), decode_start, decode_stop);
}

int pkd_run_static(const pkd_plan* p, const pkd_run_args* r) {
  if (int rc = check_run_args(p, r, PKD_STAGE_ALL); rc != PKD_OK) return rc;
  if (p->info.workspace_bytes > pkd::kStaticScratchBytes)
    return fail(PKD_ERR_WORKSPACE_TOO_SMALL,
                "the plan needs %zu bytes of scratch; the static scratch holds %zu (use pkd_run "
                "with a caller-allocated workspace)",
                p->info.workspace_bytes, pkd::kStaticScratchBytes);
  void* ws = nullptr;
  int dev = -1;
  if (const hipError_t e = pkd::static_scratch_address(&ws, &dev); e != hipSuccess)
    return fail(PKD_ERR_HIP, "static scratch of device %d: %s", dev, hipGetErrorString(e));
  // The plan's work list, merge records and zeroed fold counters, copied from
  // the plan's host image (pageable memory: the copy has read it when the
  // call returns); the previous call's contents are overwritten.
  const hipError_t e = hipMemcpyAsync(ws, p->header.data(), p->header_bytes,
                                      hipMemcpyHostToDevice, static_cast<hipStream_t>(r->stream));
  if (e != hipSuccess) return fail(PKD_ERR_HIP, "hipMemcpyAsync: %s", hipGetErrorString(e));
  return launch_run(p, r, PKD_STAGE_ALL, static_cast<char*>(ws), nullptr, nullptr);
}

int pkd_check_page_ids(const int32_t* indices, int64_t count, int32_t num_pages, void* stream,
                       int64_t* bad_out, int64_t* first_bad_out) {
  if (!bad_out) return fail(PKD_ERR_INVALID_ARGUMENT, "null output pointer");
  if (count < 0 || num_pages < 0)
    return fail(PKD_ERR_INVALID_ARGUMENT, "count and num_pages must be >= 0");
  if (count > 0 && !indices) return fail(PKD_ERR_INVALID_ARGUMENT, "null indices");
  std::vector<int32_t> ids(static_cast<size_t>(count));
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipSuccess;
  if (count > 0 &&
      (e = hipMemcpyAsync(ids.data(), indices, size_t(count) * sizeof(int32_t),
                          hipMemcpyDeviceToHost, s)) != hipSuccess)
    return fail(PKD_ERR_HIP, "hipMemcpyAsync: %s", hipGetErrorString(e));
  if ((e = hipStreamSynchronize(s)) != hipSuccess)
    return fail(PKD_ERR_HIP, "hipStreamSynchronize: %s", hipGetErrorString(e));
  int64_t bad = 0, first = -1;
  for (int64_t i = 0; i < count; ++i) {
    if (ids[size_t(i)] < 0 || ids[size_t(i)] >= num_pages) {
      if (first < 0) first = i;
      ++bad;
    }
  }
  *bad_out = bad;
  if (first_bad_out) *first_bad_out = first;
  return ok();
}

int pkd_merge_states(const pkd_merge_states_args* m) {
  if (!m) return fail(PKD_ERR_INVALID_ARGUMENT, "null argument");
  if (m->rows < 0 || m->num_heads < 1 || m->head_dim < 4 || m->head_dim % 4)
    return fail(PKD_ERR_INVALID_ARGUMENT,
                "rows must be >= 0, num_heads >= 1 and head_dim a positive multiple of 4");
  for (int dt : {m->in_dtype, m->out_dtype})
    if (dt != PKD_DTYPE_F32 && dt != PKD_DTYPE_BF16 && dt != PKD_DTYPE_F16)
      return fail(PKD_ERR_UNSUPPORTED, "merge_states takes f32, bf16 or f16 rows (dtype %d)", dt);
  if (m->rows == 0) return ok();
  if (!m->v_a || !m->s_a || !m->v_b || !m->s_b || !m->v_out)
    return fail(PKD_ERR_INVALID_ARGUMENT, "v_a, s_a, v_b, s_b and v_out must not be NULL");
  const uintptr_t in_align = m->in_dtype == PKD_DTYPE_F32 ? 16 : 8;
  const uintptr_t out_align = m->out_dtype == PKD_DTYPE_F32 ? 16 : 8;
  if (reinterpret_cast<uintptr_t>(m->v_a) % in_align ||
      reinterpret_cast<uintptr_t>(m->v_b) % in_align ||
      reinterpret_cast<uintptr_t>(m->v_out) % out_align)
    return fail(PKD_ERR_INVALID_ARGUMENT, "row pointers must be 16-byte (f32) or 8-byte (bf16) "
                                          "aligned");
  pkd::MergeStatesLaunch L;
  L.rows = m->rows;
  L.num_heads = m->num_heads;
  L.head_dim = m->head_dim;
  L.in_kind = kind_of(m->in_dtype);
  L.out_kind = kind_of(m->out_dtype);
  L.v_a = m->v_a;
  L.s_a = m->s_a;
  L.v_b = m->v_b;
  L.s_b = m->s_b;
  L.v_out = m->v_out;
  L.s_out = m->s_out;
  const hipError_t e = pkd::launch_merge_states(L, static_cast<hipStream_t>(m->stream));
  if (e != hipSuccess) return fail(PKD_ERR_HIP, "merge_states launch: %s", hipGetErrorString(e));
  return ok();
}

int pkd_stream_read(const void* buf, size_t bytes, int32_t workgroups, uint32_t* sink,
                    void* stream) {
  if (!buf || !sink) return fail(PKD_ERR_INVALID_ARGUMENT, "buf and sink must not be NULL");
  if (reinterpret_cast<uintptr_t>(buf) % 16 || bytes % 16 || bytes == 0)
    return fail(PKD_ERR_INVALID_ARGUMENT,
                "buf must be 16-byte aligned and bytes a positive multiple of 16");
  if (workgroups < 1 || workgroups > (1 << 20))
    return fail(PKD_ERR_INVALID_ARGUMENT, "workgroups must lie in [1, 2^20]");
  const hipError_t e = pkd::launch_stream_read(buf, int64_t(bytes), workgroups, sink,
                                               static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKD_ERR_HIP, "stream_read launch: %s", hipGetErrorString(e));
  return ok();
}

void pkd_plan_destroy(pkd_plan* p) {
  if (!p) return;
  pinned_release(p->staging);  // reused only after its copy has completed
  delete p;
}

}  // extern "C"
