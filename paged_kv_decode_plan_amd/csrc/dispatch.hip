// Kernel choice and launch for the decode stage.
//
// The MFMA kernel runs wherever both contractions can take bf16 operands
// exactly: bf16, e4m3, e2m1 or int4 KV with bf16 queries and head_dim 128
// (group sizes 1..32; 32 not for the 4-bit formats), and fp16 KV with fp16
// queries on fp16 MFMA.
// fp32 KV or queries, and head_dim 64, use the vector-ALU kernel, which
// handles one query token per request only. A work item of several new
// tokens of a request puts group x tokens rows (at most 32: one or two groups
// of 16 MFMA columns) on the columns; the kernel instance is the one for that
// row count (doubled for a pair of KV heads) rounded up to a power of two.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <tuple>

#include "kernel_common.h"

namespace pkd {

// Workgroup-id grouping (see decode_block) for 16-bit KV.
#ifndef PKD_XCD_GROUP_16BIT
#define PKD_XCD_GROUP_16BIT 1
#endif

static int pow2_ceil(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// Forms the MFMA kernel takes: bf16 queries over bf16, e4m3, e2m1 or int4 KV (both
// contractions on bf16 MFMA), fp16 queries over fp16 KV (fp16 MFMA).
static bool mfma_form(int kv_dtype, int q_kind) {
  return (q_kind == kQBF16 && (kv_dtype == kBF16 || kv_dtype == kE4M3 || kv_dtype == kE4M3T ||
                               kv_dtype == kE2M1 || kv_dtype == kI4)) ||
         (q_kind == kQF16 && kv_dtype == kF16);
}

static DecodeFn choose(int kv_dtype, int head_dim, int group, int rows, int q_kind,
                       int page_size, int hp = 1) {
  if ((group & (group - 1)) || rows < group || rows % group) return nullptr;
  if (hp > 1)
    return mfma_form(kv_dtype, q_kind) && hp * rows <= 32
               ? mfma_decode_kernel(kv_dtype, head_dim, pow2_ceil(hp * rows), page_size, hp)
               : nullptr;
  if (mfma_form(kv_dtype, q_kind)) {
    if (DecodeFn f = mfma_decode_kernel(kv_dtype, head_dim, pow2_ceil(rows), page_size, 1))
      return f;
  }
  // The vector-ALU kernel: one token per request, fp32 or bf16 q over fp32,
  // bf16 or e4m3 KV (per-page scales).
  if (rows != group || q_kind == kQF16 || kv_dtype == kE4M3T || kv_dtype == kF16 ||
      kv_dtype == kE2M1 || kv_dtype == kI4)
    return nullptr;
  return valu_decode_kernel(kv_dtype, head_dim, group);
}

// Dynamic LDS that caps the decode workgroups one compute unit holds at once
// at `cap` (gfx950: 160 KiB of LDS per CU): each workgroup then holds a total
// inside (160 KiB / (cap + 1), 160 KiB / cap], with margin on both sides. No
// cap (0) or a cap the other resources already impose: nothing added.
static hipError_t cap_lds(DecodeFn fn, int cap, size_t* bytes) {
  *bytes = 0;
  if (cap <= 0 || cap > 4) return hipSuccess;
  static constexpr size_t kTotal[5] = {0, 96u << 10, 72u << 10, 48u << 10, 36u << 10};
  hipFuncAttributes attr;
  if (hipError_t e = hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(fn));
      e != hipSuccess)
    return e;
  if (attr.sharedSizeBytes < kTotal[cap]) *bytes = kTotal[cap] - attr.sharedSizeBytes;
  return hipSuccess;
}

// Persistent launches of the MFMA kernel (see decode_mfma_kernel) when a
// plan has more work units than the device holds resident workgroups: for
// 16-bit and e4m3 KV with per-page scales, which run one workgroup per
// compute unit (measured on MI355X: the ragged batch 1602.6 -> 1586.6 us per
// decode launch, the fp8 batch 687.9 -> 661.3 us), not for e2m1 and int4 KV,
// which run two and three (404.3 against 397.8 us and 451.2 against
// 428.3 us), nor for e4m3 with row-wise scales, whose persistent launch was
// slower (843 against 754 us on its fp8 batch).
#ifndef PKD_PERSISTENT
#define PKD_PERSISTENT 1
#endif
#ifndef PKD_PERSISTENT_NIB4
#define PKD_PERSISTENT_NIB4 0
#endif

// Workgroups of `fn` (with `lds` bytes of dynamic LDS) the current device
// holds at once: resident per compute unit x compute units, cached per
// (device, kernel, LDS).
static hipError_t resident_workgroups(DecodeFn fn, size_t lds, int* out) {
  static std::mutex mu;
  static std::map<std::tuple<int, const void*, size_t>, int> cache;
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
  const auto key = std::make_tuple(dev, reinterpret_cast<const void*>(fn), lds);
  {
    std::lock_guard<std::mutex> lk(mu);
    if (auto it = cache.find(key); it != cache.end()) {
      *out = it->second;
      return hipSuccess;
    }
  }
  int cus = 0, per_cu = 0;
  if (hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
      e != hipSuccess)
    return e;
  if (hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, lds);
      e != hipSuccess)
    return e;
  *out = cus * per_cu;
  std::lock_guard<std::mutex> lk(mu);
  cache[key] = *out;
  return hipSuccess;
}

bool decode_supported(int kv_dtype, int head_dim, int group, int rows, int q_kind, int page_size) {
  return choose(kv_dtype, head_dim, group, rows, q_kind, page_size) != nullptr;
}

bool decode_uses_mfma(int kv_dtype, int head_dim, int group, int rows, int q_kind, int page_size) {
  return mfma_form(kv_dtype, q_kind) && rows >= group &&
         mfma_decode_kernel(kv_dtype, head_dim, pow2_ceil(rows), page_size, 1) != nullptr;
}

// KV heads per workgroup, per form (1, or 2: a pair). A pair reads a token's
// rows of both heads as one contiguous run (e2m1 rows are 64 bytes at
// head_dim 128, e4m3 128, bf16/fp16 256) and halves the workgroup count;
// measured on MI355X with one workgroup per CU, pairs are faster for bf16
// (7-8%), fp16 and e4m3 (4%) and even for e2m1.
#ifndef PKD_HEADS_E2M1
#define PKD_HEADS_E2M1 2
#endif
#ifndef PKD_HEADS_E4M3
#define PKD_HEADS_E4M3 2
#endif
#ifndef PKD_HEADS_BF16
#define PKD_HEADS_BF16 2
#endif
int decode_heads_per_wg(int kv_dtype, int head_dim, int group, int rows, int q_kind,
                        int page_size, int num_kv_heads) {
  const int hp = (kv_dtype == kE2M1 || kv_dtype == kI4) ? PKD_HEADS_E2M1
                 : (kv_dtype == kE4M3 || kv_dtype == kE4M3T) ? PKD_HEADS_E4M3
                 : (kv_dtype == kBF16 || kv_dtype == kF16) ? PKD_HEADS_BF16
                                                           : 1;
  // A pair doubles the columns: at most 16 rows per head (one column group
  // of one head, two for the pair).
  if (hp != 2 || num_kv_heads % 2 || rows > 16) return 1;
  return choose(kv_dtype, head_dim, group, rows, q_kind, page_size, 2) ? 2 : 1;
}

hipError_t launch_decode(const DecodeLaunch& L, hipStream_t stream, hipEvent_t start,
                         hipEvent_t stop) {
  const int hp = L.heads_per_wg;
  if ((hp != 1 && hp != 2) || L.num_kv_heads % hp) return hipErrorInvalidValue;
  DecodeFn fn =
      choose(L.kv_dtype, L.head_dim, L.group, L.rows, L.q_kind, 1 << L.page_size_log2, hp);
  if (!fn) return hipErrorInvalidValue;
  KernelArgs a;
  a.q = L.q;
  a.k = L.k;
  a.v = L.v;
  a.page_stride = L.page_stride;
  a.token_stride = L.token_stride;
  a.head_stride = L.head_stride;
  a.indices = L.indices;
  a.k_scale = L.k_scale;
  a.v_scale = L.v_scale;
  a.out = L.out;
  a.lse = L.lse;
  a.prior_out = L.prior_out;
  a.prior_lse = L.prior_lse;
  a.items = L.items;
  a.counts = L.counts;
  a.block_merges = L.block_merges;
  a.counters = L.counters;
  a.fuse_merge = L.fuse_merge;
  a.part_o = L.part_o;
  a.part_md = L.part_md;
  a.work = L.work;
  a.persistent = 0;
  a.num_items = L.num_items;
  a.xcd_group = (L.kv_dtype == kE4M3 || L.kv_dtype == kE4M3T || L.kv_dtype == kE2M1 ||
                 L.kv_dtype == kI4)
                    ? 8
                    : PKD_XCD_GROUP_16BIT;
  // A pair of KV heads is one workgroup "head" of 2 x group query heads.
  a.num_kv_heads = L.num_kv_heads / hp;
  a.num_qo_heads = L.num_qo_heads;
  a.group_log2 = ilog2(L.group * hp);
  a.page_size_log2 = L.page_size_log2;
  a.sm_scale_log2 = L.sm_scale_log2;
  a.q_kind = L.q_kind;
  a.out_kind = L.out_kind;
  unsigned grid = decode_grid_size(L.num_items, a.num_kv_heads, a.xcd_group);
  size_t lds = 0;
  if (hipError_t e = cap_lds(fn, L.wgs_cap, &lds); e != hipSuccess) return e;
  const bool nib4 = L.kv_dtype == kE2M1 || L.kv_dtype == kI4;
  if (PKD_PERSISTENT && (PKD_PERSISTENT_NIB4 || !nib4) && L.kv_dtype != kE4M3T && L.work &&
      decode_uses_mfma(L.kv_dtype, L.head_dim, L.group, L.rows, L.q_kind, 1 << L.page_size_log2)) {
    int resident = 0;
    if (hipError_t e = resident_workgroups(fn, lds, &resident); e != hipSuccess) return e;
    if (resident > 0 && int64_t(L.num_items) * a.num_kv_heads > resident) {
      a.persistent = 1;
      grid = unsigned(resident);
    }
  }
  if (start || stop)
    hipExtLaunchKernelGGL(fn, dim3(grid), dim3(kThreads), lds, stream, start, stop, 0, a);
  else
    hipLaunchKernelGGL(fn, dim3(grid), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

hipError_t decode_occupancy(int kv_dtype, int head_dim, int group, int rows, int q_kind,
                            int page_size, int heads_per_wg, int wgs_cap, int* wgs_per_cu) {
  DecodeFn fn = choose(kv_dtype, head_dim, group, rows, q_kind, page_size, heads_per_wg);
  if (!fn) return hipErrorInvalidValue;
  size_t lds = 0;
  if (hipError_t e = cap_lds(fn, wgs_cap, &lds); e != hipSuccess) return e;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(wgs_per_cu, fn, kThreads, lds);
}

}  // namespace pkd
