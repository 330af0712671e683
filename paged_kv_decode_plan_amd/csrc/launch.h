// Internal interface between the C-ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pkd {

// KV element formats as the kernels see them: kE4M3T is e4m3 with one scale
// per (token, KV head) instead of one per (page, KV head); kE2M1 is FP4 E2M1
// and kI4 two's-complement int4, both two elements per byte, with one scale
// per (KV head, channel).
enum : int { kF32 = 0, kBF16 = 1, kE4M3 = 2, kE4M3T = 3, kF16 = 4, kE2M1 = 5, kI4 = 6 };
// Query / output element formats.
enum : int { kQF32 = 0, kQBF16 = 1, kQF16 = 2 };

// Device-side layout of one work item (32 bytes): pages
// [page_begin, page_begin + ceil(kv_len / page_size)) of the page table for
// the q rows [q_row, q_row + q_len). kv_len counts only tokens some row of
// the block sees; row i sees min(kv_len, visible + i) of them (the causal
// limit of several new tokens per request; one token sees them all).
struct DeviceItem {
  int32_t page_begin;
  int32_t kv_len;
  int32_t partial_slot;  // partial-state row of q row q_row; -1: write the output
  int32_t q_row;
  int32_t q_len;
  int32_t visible;
  int32_t block_merge;  // split item: its (request, query block)'s merge record; else -1
  int32_t pad;
};

// Device-side record of one merge (16 bytes): output row out_row folds the
// partial-state rows first + c * stride for c in [0, count).
struct MergeTask {
  int32_t out_row;
  int32_t first;
  int32_t count;
  int32_t stride;
};

struct DecodeLaunch {
  int kv_dtype = 0;
  int head_dim = 0;
  int group = 0;
  int rows = 0;  // query rows per work item and KV head: group x query tokens per item
  int heads_per_wg = 1;  // KV heads per decode workgroup (see decode_heads_per_wg)
  int wgs_cap = 0;  // at most this many decode workgroups per compute unit (0: no cap)
  int num_items = 0;
  int num_kv_heads = 0;
  int num_qo_heads = 0;
  int page_size_log2 = 0;
  float sm_scale_log2 = 0.f;  // sm_scale * log2(e)
  int q_kind = 0;    // kQF32, kQBF16 or kQF16
  int out_kind = 0;  // kQF32, kQBF16 or kQF16
  const void* q = nullptr;
  const void* k = nullptr;
  const void* v = nullptr;
  int64_t page_stride = 0;
  int64_t token_stride = 0;
  int64_t head_stride = 0;
  const int32_t* indices = nullptr;
  const float* k_scale = nullptr;
  const float* v_scale = nullptr;
  void* out = nullptr;
  float* lse = nullptr;
  // Another normalised result of the same rows (fp32 rows, natural-log LSE)
  // to merge into the output as it is written; nullptr: none.
  const float* prior_out = nullptr;
  const float* prior_lse = nullptr;
  const DeviceItem* items = nullptr;
  float* part_o = nullptr;   // [num_partials, Hq, head_dim]
  float* part_md = nullptr;  // [num_partials, Hq, 2]: (m in log2 units, d)
  int num_split = 0;                       // merge tasks
  const MergeTask* merge_tasks = nullptr;  // [num_split]
  // Fixed-capacity plans: {work items, merge tasks} of the uploaded plan, read
  // by the kernels (num_items / num_split are then the capacities). nullptr:
  // the launch is sized exactly.
  const int32_t* counts = nullptr;
  // Two counters, zero between launches, for a persistent launch of the MFMA
  // kernel (work units taken, workgroups finished); nullptr: plain launches.
  int32_t* work = nullptr;
  // Merge folded into the decode kernel: one record per (split request, query
  // block) (out_row = its first q row, count = chunks, stride = q_r) and one
  // arrival counter per (record, KV head), zero between runs.
  int fuse_merge = 0;
  const MergeTask* block_merges = nullptr;
  int32_t* counters = nullptr;
};

// `rows` is group x (query tokens per work item); rows > group (several new
// tokens per request) is served by the MFMA kernel only.
bool decode_supported(int kv_dtype, int head_dim, int group, int rows, int q_kind, int page_size);
bool decode_uses_mfma(int kv_dtype, int head_dim, int group, int rows, int q_kind, int page_size);
// KV heads one decode workgroup handles: 2 (a pair, read as one contiguous
// run per token) on the MFMA path where the KV head count is even, a head has
// at most 16 rows per work item (the pair's then fill at most two 16-column
// groups) and pages hold at least 16 tokens; otherwise 1.
int decode_heads_per_wg(int kv_dtype, int head_dim, int group, int rows, int q_kind,
                        int page_size, int num_kv_heads);
// start / stop: events the kernel's dispatch records as it begins and
// completes (nullptr: a plain launch).
hipError_t launch_decode(const DecodeLaunch& a, hipStream_t stream, hipEvent_t start = nullptr,
                         hipEvent_t stop = nullptr);
hipError_t launch_merge(const DecodeLaunch& a, hipStream_t stream);
hipError_t decode_occupancy(int kv_dtype, int head_dim, int group, int rows, int q_kind,
                            int page_size, int heads_per_wg, int wgs_cap, int* wgs_per_cu);

struct MergeStatesLaunch {
  int64_t rows = 0;
  int num_heads = 0;
  int head_dim = 0;
  int in_kind = 0;   // kQF32, kQBF16 or kQF16
  int out_kind = 0;
  const void* v_a = nullptr;
  const float* s_a = nullptr;
  const void* v_b = nullptr;
  const float* s_b = nullptr;
  void* v_out = nullptr;
  float* s_out = nullptr;
};
hipError_t launch_merge_states(const MergeStatesLaunch& a, hipStream_t stream);

// Streaming read of `bytes` (a multiple of 16) at `buf` (16-byte aligned) by
// `workgroups` workgroups of four wavefronts; `sink` receives 4 words per
// workgroup.
hipError_t launch_stream_read(const void* buf, int64_t bytes, int workgroups, uint32_t* sink,
                              hipStream_t stream);

// Static device scratch of the entry point that allocates nothing: its size,
// and its address on the current device (*device receives that device).
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
hipError_t static_scratch_address(void** ptr, int* device);

}  // namespace pkd
