// Merge of split-KV partial states, for gfx950.
//
// Folds the partial (m, d, o) states that the decode kernel wrote for the
// chunks of one request with the online-softmax merge rule of "FlashDecoding +
// FlashInfer — the decode-time attention story", §"FlashDecoding — the
// split-KV trick", then normalises: out = o / d, lse = m + ln d.
//
// One workgroup per (split request, query head). All lanes first find the
// largest m over the request's partials; then each wavefront folds every
// fourth partial (each lane owning head_dim / 64 output dims, loads unrolled
// four deep), and the four wavefront sums are added in shared memory. With
// the common maximum the fold is a plain weighted sum, so its order does not
// change the result beyond rounding, and the result is the same on every run.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernel_common.h"

namespace pkd {

namespace {

struct MergeArgs {
  const float* part_o;
  const float* part_md;
  const int32_t* split_requests;
  const int32_t* merge_indptr;
  void* out;
  float* lse;
  int num_qo_heads;
  int out_bf16;
};

constexpr int kMergeWaves = 4;

template <int D>
__global__ __launch_bounds__(kMergeWaves * 64) void merge_kernel(MergeArgs a) {
  constexpr int PER = D / 64;  // output dims per lane
  __shared__ float so[kMergeWaves][D];
  __shared__ float sd[kMergeWaves];
  const int hq = blockIdx.x % a.num_qo_heads;
  const int r = a.split_requests[blockIdx.x / a.num_qo_heads];
  const int b = a.merge_indptr[r];
  const int e = a.merge_indptr[r + 1];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t H = a.num_qo_heads;

  float M = -INFINITY;
  for (int i = b + lane; i < e; i += 64) M = fmaxf(M, a.part_md[(int64_t(i) * H + hq) * 2]);
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) M = fmaxf(M, __shfl_xor(M, s, 64));

  float O[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) O[k] = 0.f;
  float Dn = 0.f;
  constexpr int kUnroll = 4;
  for (int i0 = b + wave; i0 < e; i0 += kMergeWaves * kUnroll) {
    float m[kUnroll], d[kUnroll], o[kUnroll][PER];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int i = i0 + u * kMergeWaves;
      m[u] = -INFINITY;
      d[u] = 0.f;
#pragma unroll
      for (int k = 0; k < PER; ++k) o[u][k] = 0.f;
      if (i < e) {
        const int64_t prow = int64_t(i) * H + hq;
        m[u] = a.part_md[prow * 2];
        d[u] = a.part_md[prow * 2 + 1];
#pragma unroll
        for (int k = 0; k < PER; ++k) o[u][k] = a.part_o[prow * D + lane * PER + k];
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float sc = exp2f(m[u] - M);
      Dn = fmaf(d[u], sc, Dn);
#pragma unroll
      for (int k = 0; k < PER; ++k) O[k] = fmaf(o[u][k], sc, O[k]);
    }
  }
#pragma unroll
  for (int k = 0; k < PER; ++k) so[wave][lane * PER + k] = O[k];
  if (lane == 0) sd[wave] = Dn;
  __syncthreads();
  if (threadIdx.x < D) {
    const int dd = threadIdx.x;
    float Ot = 0.f, Dt = 0.f;
#pragma unroll
    for (int w = 0; w < kMergeWaves; ++w) {
      Ot += so[w][dd];
      Dt += sd[w];
    }
    const int64_t row = int64_t(r) * H + hq;
    const float val = Ot / Dt;
    if (a.out_bf16)
      static_cast<uint16_t*>(a.out)[row * D + dd] = float_to_bf16_rne(val);
    else
      static_cast<float*>(a.out)[row * D + dd] = val;
    if (a.lse && dd == 0) a.lse[row] = (M + log2f(Dt)) * kLn2;
  }
}

}  // namespace

hipError_t launch_merge(const DecodeLaunch& L, hipStream_t stream) {
  if (L.num_split == 0) return hipSuccess;
  MergeArgs a;
  a.part_o = L.part_o;
  a.part_md = L.part_md;
  a.split_requests = L.split_requests;
  a.merge_indptr = L.merge_indptr;
  a.out = L.out;
  a.lse = L.lse;
  a.num_qo_heads = L.num_qo_heads;
  a.out_bf16 = L.out_bf16;
  const unsigned grid = unsigned(L.num_split) * unsigned(L.num_qo_heads);
  const dim3 block(kMergeWaves * 64);
  if (L.head_dim == 64)
    hipLaunchKernelGGL(merge_kernel<64>, dim3(grid), block, 0, stream, a);
  else if (L.head_dim == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3(grid), block, 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pkd
