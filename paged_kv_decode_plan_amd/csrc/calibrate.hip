// Plain streaming read of device memory, for gfx950: the calibration that
// puts the decode kernels' KV-read rate beside what one kernel can pull from
// HBM on the same device (the pages rate decode kernels by the fraction of
// memory bandwidth they reach: "Attention Kernel Comparison: FlashAttention
// vs FlashInfer vs xformers vs Triton", opening paragraphs).
//
// Each workgroup (four wavefronts) walks 32 KiB blocks of the buffer in a
// grid-stride loop: per block every lane issues kLoads 16-byte loads, lane l of
// wavefront w reading unit (u * 256 + 64 * w + l), so that every load
// instruction of a wavefront covers 1 KiB of consecutive bytes and a
// wavefront keeps 8 KiB in flight. The loads are non-temporal (the data is
// read once): measured on MI355X with one workgroup per compute unit, that
// policy reads 7.3 TB/s where the default one reads 6.4 TB/s, whether or not
// the next block's loads are issued before this block's are consumed. The
// loaded words are folded with XOR and each wavefront stores its fold (one
// word), so the loads cannot be dropped. The caller picks the grid (a
// multiple of the compute-unit count: one to a few workgroups per compute
// unit).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "launch.h"

namespace pkd {

namespace {

constexpr int kCalThreads = 256;
constexpr int kLoads = 8;

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

__global__ __launch_bounds__(kCalThreads) void stream_read_kernel(const u32x4_t* p, int64_t units,
                                                                  uint32_t* sink) {
  constexpr int64_t kBlock = int64_t(kCalThreads) * kLoads;  // 16-byte units per block
  uint32_t acc = 0;
  for (int64_t base = int64_t(blockIdx.x) * kBlock; base < units;
       base += int64_t(gridDim.x) * kBlock) {
    u32x4_t v[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int64_t i = base + int64_t(u) * kCalThreads + threadIdx.x;
      v[u] = i < units ? __builtin_nontemporal_load(p + i) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kLoads; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0) sink[int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6)] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, int64_t bytes, int workgroups, uint32_t* sink,
                              hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(unsigned(workgroups)), dim3(kCalThreads), 0, stream,
                     static_cast<const u32x4_t*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace pkd
