// Merge of two normalised attention results over disjoint token sets, for
// gfx950: the combining step of cascade attention (shared-prefix level and
// per-request suffix level).
//
// A result (v, s) of a query row (output row v, natural-log log-sum-exp s) is
// the softmax state (m = s, d = 1, o = v); two states merge with the rule of
// "FlashDecoding + FlashInfer — the decode-time attention story",
// §"FlashDecoding — the split-KV trick": with m = max(s_a, s_b) and
// w_x = e^(s_x - m), v = (w_a v_a + w_b v_b) / (w_a + w_b) and
// s = m + ln(w_a + w_b). s = -inf (no tokens) has weight 0.
//
// Elementwise and HBM-bound: one thread per four consecutive dims of one
// (row, head), vector loads and stores, a grid-stride loop over the rows.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernel_common.h"

namespace pkd {

namespace {

constexpr int kMsThreads = 256;
constexpr float kLog2e = 1.44269504088896340736f;

__device__ inline float4 load4(const void* p, int64_t i, int kind) {
  if (kind == kQBF16) {
    const uint2 w = reinterpret_cast<const uint2*>(p)[i];
    return float4{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                  __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
  }
  if (kind == kQF16) {
    const uint2 w = reinterpret_cast<const uint2*>(p)[i];
    auto h = [](uint32_t b) { return float(__builtin_bit_cast(_Float16, uint16_t(b))); };
    return float4{h(w.x & 0xffffu), h(w.x >> 16), h(w.y & 0xffffu), h(w.y >> 16)};
  }
  return reinterpret_cast<const float4*>(p)[i];
}

__global__ __launch_bounds__(kMsThreads) void merge_states_kernel(MergeStatesLaunch a) {
  const int quads = a.head_dim / 4;
  const int64_t total = a.rows * a.num_heads * quads;
  for (int64_t i = int64_t(blockIdx.x) * kMsThreads + threadIdx.x; i < total;
       i += int64_t(gridDim.x) * kMsThreads) {
    const int64_t rh = i / quads;  // (row, head)
    const float sa = a.s_a[rh], sb = a.s_b[rh];
    const float m = fmaxf(sa, sb);
    const float wa = sa == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((sa - m) * kLog2e);
    const float wb = sb == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((sb - m) * kLog2e);
    const float wsum = wa + wb;
    const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
    const float4 va = load4(a.v_a, i, a.in_kind);
    const float4 vb = load4(a.v_b, i, a.in_kind);
    const float4 v = {(va.x * wa + vb.x * wb) * inv, (va.y * wa + vb.y * wb) * inv,
                      (va.z * wa + vb.z * wb) * inv, (va.w * wa + vb.w * wb) * inv};
    if (a.out_kind != kQF32) {
      reinterpret_cast<uint2*>(a.v_out)[i] = pack4_16(v.x, v.y, v.z, v.w, a.out_kind);
    } else {
      reinterpret_cast<float4*>(a.v_out)[i] = v;
    }
    if (a.s_out && i % quads == 0) a.s_out[rh] = wsum > 0.f ? m + logf(wsum) : -INFINITY;
  }
}

}  // namespace

hipError_t launch_merge_states(const MergeStatesLaunch& a, hipStream_t stream) {
  const int64_t total = a.rows * a.num_heads * (a.head_dim / 4);
  if (total == 0) return hipSuccess;
  const int64_t blocks = (total + kMsThreads - 1) / kMsThreads;
  const unsigned grid = unsigned(blocks < 65536 ? blocks : 65536);
  hipLaunchKernelGGL(merge_states_kernel, dim3(grid), dim3(kMsThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkd
