// Merge of split-KV partial states, for gfx950.
//
// Folds the partial (m, d, o) states that the decode kernel wrote for the
// chunks of one request with the online-softmax merge rule of "FlashDecoding +
// FlashInfer — the decode-time attention story", §"FlashDecoding — the
// split-KV trick": m = max(m_a, m_b), d and o rescaled by exp(m_a - m) and
// exp(m_b - m) and added; then normalises: out = o / d, lse = m + ln d
// (partial m is kept in log2 units, so the kernel uses exp2).
//
// One workgroup per (merge task, query head): a task is one q row of a split
// request, whose partial states are the rows first + c * stride, c < count
// (stride 1 with one query token per request; with several new tokens the
// chunks' rows of one token are that many apart). Thread (s, p) owns output
// dims 4p..4p+3 and folds the partials c congruent to s modulo S
// (S = 512 / (head_dim / 4) subsets), four at a time with all their loads
// issued first; the S subset states are then merged through shared memory.
// The empty state (m = -inf, d = 0: a chunk wholly past a new token's causal
// limit) is the identity of the fold. The task record comes from the plan in
// one 16-byte load.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernel_common.h"

namespace pkd {

namespace {

struct MergeArgs {
  const float* part_o;
  const float* part_md;
  const MergeTask* tasks;
  const int32_t* counts;  // fixed-capacity plan: counts[1] merge tasks are live
  void* out;
  float* lse;
  const float* prior_out;  // another result of the same rows to merge in, or nullptr
  const float* prior_lse;
  int num_qo_heads;
  int out_kind;  // kQF32, kQBF16 or kQF16
};

constexpr int kMergeThreads = 512;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeArgs a) {
  constexpr int kQuads = D / 4;                  // threads per subset (four dims each)
  constexpr int kSub = kMergeThreads / kQuads;   // partial subsets
  __shared__ float sm[kSub], sd[kSub];
  __shared__ float4 so[kSub][kQuads];
  const int H = a.num_qo_heads;
  if (a.counts && int(blockIdx.x / H) >= a.counts[1]) return;  // past the plan's tasks
  const MergeTask t = a.tasks[blockIdx.x / H];
  const int h = blockIdx.x % H;
  const int sub = threadIdx.x / kQuads;
  const int qd = threadIdx.x % kQuads;

  const float2* md = reinterpret_cast<const float2*>(a.part_md);
  const float4* po = reinterpret_cast<const float4*>(a.part_o);
  float M = -INFINITY, Dn = 0.f;
  float4 O = {0.f, 0.f, 0.f, 0.f};
  constexpr int kU = 4;
  for (int c0 = sub; c0 < t.count; c0 += kU * kSub) {
    float2 mdv[kU];
    float4 ov[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int c = min(c0 + u * kSub, t.count - 1);  // a clamped repeat is skipped below
      const int64_t row = (int64_t(t.first) + int64_t(c) * t.stride) * H + h;
      mdv[u] = md[row];
      ov[u] = po[row * kQuads + qd];
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (c0 + u * kSub < t.count) {
        const float m_new = fmaxf(M, mdv[u].x);
        // 0 on the first partial (M = -inf), and for an empty partial
        const float sa = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - m_new);
        const float sb = mdv[u].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mdv[u].x - m_new);
        Dn = Dn * sa + mdv[u].y * sb;
        O.x = O.x * sa + ov[u].x * sb;
        O.y = O.y * sa + ov[u].y * sb;
        O.z = O.z * sa + ov[u].z * sb;
        O.w = O.w * sa + ov[u].w * sb;
        M = m_new;
      }
    }
  }
  if (qd == 0) {
    sm[sub] = M;
    sd[sub] = Dn;
  }
  so[sub][qd] = O;
  __syncthreads();
  if (sub == 0) {
    float Mt = sm[0];
#pragma unroll
    for (int k = 1; k < kSub; ++k) Mt = fmaxf(Mt, sm[k]);
    float Dt = 0.f;
    float4 A = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kSub; ++k) {
      const float w = sm[k] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sm[k] - Mt);  // empty subset
      Dt += sd[k] * w;
      A.x += so[k][qd].x * w;
      A.y += so[k][qd].y * w;
      A.z += so[k][qd].z * w;
      A.w += so[k][qd].w * w;
    }
    const int64_t row = int64_t(t.out_row) * H + h;
    if (a.prior_out) {
      const PriorWeights pw = fold_prior(Mt, Dt, a.prior_lse[row]);
      A = fold_prior4(A, reinterpret_cast<const float4*>(a.prior_out)[row * kQuads + qd], pw);
    }
    const float inv = Dt > 0.f ? 1.0f / Dt : 0.f;
    if (a.out_kind != kQF32) {
      reinterpret_cast<uint2*>(a.out)[row * kQuads + qd] =
          pack4_16(A.x * inv, A.y * inv, A.z * inv, A.w * inv, a.out_kind);
    } else {
      reinterpret_cast<float4*>(a.out)[row * kQuads + qd] =
          float4{A.x * inv, A.y * inv, A.z * inv, A.w * inv};
    }
    if (a.lse && qd == 0) a.lse[row] = Dt > 0.f ? (Mt + log2f(Dt)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_merge(const DecodeLaunch& L, hipStream_t stream) {
  if (L.num_split == 0) return hipSuccess;
  MergeArgs a;
  a.part_o = L.part_o;
  a.part_md = L.part_md;
  a.tasks = L.merge_tasks;
  a.counts = L.counts;
  a.out = L.out;
  a.lse = L.lse;
  a.prior_out = L.prior_out;
  a.prior_lse = L.prior_lse;
  a.num_qo_heads = L.num_qo_heads;
  a.out_kind = L.out_kind;
  const unsigned grid = unsigned(L.num_split) * unsigned(L.num_qo_heads);
  if (L.head_dim == 64)
    hipLaunchKernelGGL(merge_kernel<64>, dim3(grid), dim3(kMergeThreads), 0, stream, a);
  else if (L.head_dim == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3(grid), dim3(kMergeThreads), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkd
