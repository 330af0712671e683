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
// Elementwise and HBM-bound. A workgroup takes a tile of kMsTile (row, head)
// pairs: thread t < kMsTile reads the two LSEs of pair t, keeps the merged LSE
// and shares the two weights through LDS; after a barrier every thread
// merges four consecutive dims at a time over the tile's rows (vector loads
// and stores, consecutive threads on consecutive dims), and thread t then
// writes pair t's LSE. Each LSE is read and written by one thread and each
// output element by the thread that read its inputs, and no other workgroup
// touches the tile, so the output may alias an input (an in-place merge) for
// every head_dim. Tiles are visited by a grid-stride loop.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernel_common.h"

namespace pkd {

namespace {

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

constexpr int kMsThreads = 256;
constexpr int kMsTile = 64;  // (row, head) pairs per workgroup tile

__global__ __launch_bounds__(kMsThreads) void merge_states_kernel(MergeStatesLaunch a) {
  __shared__ float s_wa[kMsTile], s_wb[kMsTile];
  const int quads = a.head_dim / 4;
  const int64_t pairs = a.rows * a.num_heads;
  for (int64_t base = int64_t(blockIdx.x) * kMsTile; base < pairs;
       base += int64_t(gridDim.x) * kMsTile) {
    const int n = int(pairs - base < kMsTile ? pairs - base : kMsTile);
    float s_new = -INFINITY;
    if (int(threadIdx.x) < n) {
      const int64_t rh = base + threadIdx.x;
      const float sa = a.s_a[rh], sb = a.s_b[rh];
      const float m = fmaxf(sa, sb);
      const float wa = sa == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((sa - m) * kLog2e);
      const float wb = sb == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((sb - m) * kLog2e);
      const float wsum = wa + wb;
      const float inv = wsum > 0.f ? 1.0f / wsum : 0.f;
      s_wa[threadIdx.x] = wa * inv;
      s_wb[threadIdx.x] = wb * inv;
      if (wsum > 0.f) s_new = m + logf(wsum);
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < n * quads; idx += kMsThreads) {
      const int t = idx / quads;
      const int64_t i = base * quads + idx;  // quad index over [rows, heads, head_dim / 4]
      const float wa = s_wa[t], wb = s_wb[t];
      const float4 va = load4(a.v_a, i, a.in_kind);
      const float4 vb = load4(a.v_b, i, a.in_kind);
      const float4 v = {va.x * wa + vb.x * wb, va.y * wa + vb.y * wb, va.z * wa + vb.z * wb,
                        va.w * wa + vb.w * wb};
      if (a.out_kind != kQF32) {
        reinterpret_cast<uint2*>(a.v_out)[i] = pack4_16(v.x, v.y, v.z, v.w, a.out_kind);
      } else {
        reinterpret_cast<float4*>(a.v_out)[i] = v;
      }
    }
    if (a.s_out && int(threadIdx.x) < n) a.s_out[base + threadIdx.x] = s_new;
    __syncthreads();  // the weights of this tile are read before the next tile's
  }
}

}  // namespace

hipError_t launch_merge_states(const MergeStatesLaunch& a, hipStream_t stream) {
  const int64_t pairs = a.rows * a.num_heads;
  if (pairs == 0) return hipSuccess;
  const int64_t tiles = (pairs + kMsTile - 1) / kMsTile;
  const unsigned grid = unsigned(tiles < 65536 ? tiles : 65536);
  hipLaunchKernelGGL(merge_states_kernel, dim3(grid), dim3(kMsThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkd
