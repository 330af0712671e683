// Device-side pieces shared by the decode kernels: kernel arguments, bf16
// rounding, and the end-of-workgroup merge of per-wavefront softmax states.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "launch.h"

namespace pkd {

constexpr int kWaves = 4;               // wavefronts per decode workgroup
constexpr int kThreads = kWaves * 64;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

struct KernelArgs {
  const void* q;
  const void* k;
  const void* v;
  int64_t page_stride;
  int64_t token_stride;
  int64_t head_stride;
  const int32_t* indices;
  const float* k_scale;
  const float* v_scale;
  void* out;
  float* lse;
  const float* prior_out;  // another result of the same rows to merge in, or nullptr
  const float* prior_lse;
  const DeviceItem* items;
  const int32_t* counts;  // nullptr, or {work items, merge tasks} of the uploaded plan
  const MergeTask* block_merges;  // fused merge records (fuse_merge only)
  int32_t* counters;              // fused merge arrival counters, [record][KV head]
  int fuse_merge;
  float* part_o;
  float* part_md;
  // Persistent launch (persistent = 1): the grid is the device's resident
  // workgroups and each workgroup takes work units (item, KV head) in plan
  // order from work[0]; work[1] counts finished workgroups, and the last one
  // resets both to zero for the next launch.
  int* work;
  int persistent;
  int num_items;
  int xcd_group;  // workgroup-id grouping g (see decode_block)
  int num_kv_heads;
  int num_qo_heads;
  int group_log2;  // query heads per KV head (a power of two), as log2
  int page_size_log2;
  float sm_scale_log2;  // logit scale times log2(e): scores are kept in log2 units
  int q_kind;    // kQF32, kQBF16 or kQF16
  int out_kind;  // kQF32, kQBF16 or kQF16
};

using DecodeFn = void (*)(KernelArgs);

// The hardware hands consecutive workgroup ids to the 8 XCDs round robin
// (id % 8), each XCD with its own L2. With grouping g = 8, decode workgroups
// are numbered so that all KV heads of one item run on the same XCD and share
// its L2 lines of page ids, query rows and per-(page, head) scales:
//   id = g * (Hkv * (item / g) + kvh) + item % g;
// g = 1 is the plain id = item * Hkv + kvh, which spreads the heads of a page
// over the XCDs. Items start in plan order either way. The grid covers the
// item count rounded up to a multiple of g; ids past the last item do nothing.
// (Measured on MI355X: g = 8 is faster for e4m3 KV, whose scale lines the
// heads share, and g = 1 for bf16 KV.)
__host__ __device__ inline unsigned decode_grid_size(int num_items, int num_kv_heads, int g) {
  return unsigned((num_items + g - 1) / g) * unsigned(g) * unsigned(num_kv_heads);
}

__device__ inline void decode_block(int num_kv_heads, int g, int* item, int* kvh) {
  const int id = int(blockIdx.x);
  *item = g * (id / (g * num_kv_heads)) + id % g;
  *kvh = (id / g) % num_kv_heads;
}

// Work items of this launch: the grid's count, or, for a fixed-capacity plan
// (grid sized by its capacity), the count its upload wrote to the workspace.
__device__ inline int launch_items(const KernelArgs& a) {
  return a.counts ? a.counts[0] : a.num_items;
}

__device__ inline float bf16_bits_to_float(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

__device__ inline uint16_t float_to_f16_rne(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));  // round to nearest even
}

__device__ inline uint16_t float_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Four values rounded to the 16-bit output format (kQBF16 or kQF16), packed.
__device__ inline uint2 pack4_16(float x, float y, float z, float w, int kind) {
  if (kind == kQF16)
    return uint2{uint32_t(float_to_f16_rne(x)) | (uint32_t(float_to_f16_rne(y)) << 16),
                 uint32_t(float_to_f16_rne(z)) | (uint32_t(float_to_f16_rne(w)) << 16)};
  return uint2{uint32_t(float_to_bf16_rne(x)) | (uint32_t(float_to_bf16_rne(y)) << 16),
               uint32_t(float_to_bf16_rne(z)) | (uint32_t(float_to_bf16_rne(w)) << 16)};
}

// threadIdx.x through an empty asm statement: the epilogues below run once
// per work unit of a persistent workgroup, and values derived from an opaque
// index are not computed once for all units and held in registers.
__device__ inline int opaque_tid() {
  int t = int(threadIdx.x);
  asm volatile("" : "+v"(t));
  return t;
}

// Fold another normalised result of the same row (output value v_p per dim,
// natural-log LSE lse_p; the cascade's other level) into the state (M in
// log2 units, d, o) about to be written: the prior is the state
// (lse_p * log2 e, 1, v_p) and the rule is the online-softmax merge. Returns
// the weights of the state's o and of v_p and updates M and d; both sides
// empty leaves d = 0 (the row is then 0 with LSE -inf).
struct PriorWeights {
  float self, prior;
};
__device__ inline PriorWeights fold_prior(float& M, float& Dn, float lse_p) {
  const float mp = lse_p * kLog2e;
  const float mn = fmaxf(M, mp);
  PriorWeights w;
  w.self = M == -INFINITY ? 0.f : exp2f(M - mn);
  w.prior = mp == -INFINITY ? 0.f : exp2f(mp - mn);
  Dn = Dn * w.self + w.prior;
  M = mn;
  return w;
}
__device__ inline float4 fold_prior4(float4 O, float4 vp, const PriorWeights& w) {
  return float4{O.x * w.self + vp.x * w.prior, O.y * w.self + vp.y * w.prior,
                O.z * w.self + vp.z * w.prior, O.w * w.self + vp.w * w.prior};
}

// The merge of a split request, folded into the decode kernel: every
// workgroup of a chunk counts itself in with one atomic add on the (request,
// query block, KV head) counter, made by one thread after a workgroup
// barrier and with release ordering at device scope, which publishes every
// wavefront's partial states; the one that completes the count is the last,
// and after an acquire fence it folds the chunks' partial states of its rows
// with the online-softmax rule (chunks in order, so the result does not
// depend on which workgroup finishes last), writes the output rows and LSE,
// and resets the counter for the next run. Called by every thread of the
// workgroup. On gfx950 a device-scope release writes back the XCD's L2 and an
// acquire invalidates it, each a few microseconds: one thread does each, once
// per workgroup (a fence in every thread took four of each per workgroup).
template <int D>
__device__ inline void merge_if_last(const KernelArgs& a, const DeviceItem& it, int kvh,
                                     int nthreads) {
  __shared__ int s_last;
  const MergeTask mt = a.block_merges[it.block_merge];
  int32_t* counter = a.counters + int64_t(it.block_merge) * a.num_kv_heads + kvh;
  const int tid = opaque_tid();
  __syncthreads();  // every wavefront's partial states before thread 0's arrival
  if (tid == 0) {
    const int prior = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = prior == mt.count - 1;
    // the other chunks' partial states after their arrivals
    if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  const int gmask = (1 << a.group_log2) - 1;
  const int rows = it.q_len << a.group_log2;
  constexpr int kQuads = D / 4;
  constexpr int kU = 8;  // chunks whose loads are in flight together
  const float2* md = reinterpret_cast<const float2*>(a.part_md);
  const float4* po = reinterpret_cast<const float4*>(a.part_o);
  for (int idx = tid; idx < rows * kQuads; idx += nthreads) {
    const int h = idx / kQuads;
    const int qd = idx % kQuads;
    const int i = h >> a.group_log2;
    const int hq = (kvh << a.group_log2) + (h & gmask);
    float M = -INFINITY, Dn = 0.f;
    float4 O = {0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < mt.count; c0 += kU) {
      float2 st[kU];
      float4 ov[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int c = min(c0 + u, mt.count - 1);  // a clamped repeat is skipped below
        const int64_t prow =
            (int64_t(mt.first) + int64_t(c) * mt.stride + i) * a.num_qo_heads + hq;
        st[u] = md[prow];
        ov[u] = po[prow * kQuads + qd];
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (c0 + u < mt.count) {
          const float m_new = fmaxf(M, st[u].x);
          const float sa = M == -INFINITY ? 0.f : exp2f(M - m_new);
          const float sb = st[u].x == -INFINITY ? 0.f : exp2f(st[u].x - m_new);
          Dn = Dn * sa + st[u].y * sb;
          O.x = O.x * sa + ov[u].x * sb;
          O.y = O.y * sa + ov[u].y * sb;
          O.z = O.z * sa + ov[u].z * sb;
          O.w = O.w * sa + ov[u].w * sb;
          M = m_new;
        }
      }
    }
    const int64_t row = int64_t(mt.out_row + i) * a.num_qo_heads + hq;
    if (a.prior_out) {
      const PriorWeights pw = fold_prior(M, Dn, a.prior_lse[row]);
      O = fold_prior4(O, reinterpret_cast<const float4*>(a.prior_out)[row * kQuads + qd], pw);
    }
    const float inv = Dn > 0.f ? 1.0f / Dn : 0.f;
    if (a.out_kind != kQF32) {
      reinterpret_cast<uint2*>(a.out)[row * kQuads + qd] =
          pack4_16(O.x * inv, O.y * inv, O.z * inv, O.w * inv, a.out_kind);
    } else {
      reinterpret_cast<float4*>(a.out)[row * kQuads + qd] =
          float4{O.x * inv, O.y * inv, O.z * inv, O.w * inv};
    }
    if (a.lse && qd == 0) a.lse[row] = Dn > 0.f ? (M + log2f(Dn)) * kLn2 : -INFINITY;
  }
  if (tid == 0) *counter = 0;
}

// Shared-memory image of the wavefronts' states for the final merge.
template <int G, int D>
struct WaveStates {
  float o[kWaves][G][D];  // unnormalised sums of p * v, relative to m
  float m[kWaves][G];     // running max, log2 units (-inf: the wavefront saw no token)
  float d[kWaves][G];     // sum of p
};

// Merge the kWaves states of every row (query token i, query head hh of the
// group; row = i * group + hh) with the online-softmax rule and write either
// the normalised output row (and its log-sum-exp) or, for a split request,
// the partial state (m, d, o). A row none of whose tokens were seen here (a
// chunk past a new token's causal limit) gives the empty state (-inf, 0, 0).
// Must be called by all threads of the workgroup after a barrier.
template <int G, int D>
__device__ inline void finish_workgroup(const WaveStates<G, D>& s, const KernelArgs& a,
                                        const DeviceItem& it, int kvh) {
  const int gmask = (1 << a.group_log2) - 1;
  for (int idx = opaque_tid(); idx < G * D; idx += kThreads) {
    const int h = idx / D;
    const int d = idx % D;
    const int i = h >> a.group_log2;
    if (i >= it.q_len) break;  // rows are in order: every later one is padding too
    float M = s.m[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, s.m[w][h]);
    float O = 0.f, Dn = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = s.m[w][h];
      const float sc = mw == -INFINITY ? 0.f : exp2f(mw - M);  // a wavefront without tokens
      O = fmaf(s.o[w][h][d], sc, O);
      Dn = fmaf(s.d[w][h], sc, Dn);
    }
    const int hq = (kvh << a.group_log2) + (h & gmask);
    const int64_t row = int64_t(it.q_row + i) * a.num_qo_heads + hq;
    if (it.partial_slot < 0) {
      if (a.prior_out) {
        const PriorWeights pw = fold_prior(M, Dn, a.prior_lse[row]);
        O = O * pw.self + a.prior_out[row * D + d] * pw.prior;
      }
      const float val = Dn > 0.f ? O / Dn : 0.f;
      if (a.out_kind == kQBF16)
        static_cast<uint16_t*>(a.out)[row * D + d] = float_to_bf16_rne(val);
      else if (a.out_kind == kQF16)
        static_cast<uint16_t*>(a.out)[row * D + d] = float_to_f16_rne(val);
      else
        static_cast<float*>(a.out)[row * D + d] = val;
      if (a.lse && d == 0) a.lse[row] = Dn > 0.f ? (M + log2f(Dn)) * kLn2 : -INFINITY;
    } else {
      const int64_t prow = int64_t(it.partial_slot + i) * a.num_qo_heads + hq;
      a.part_o[prow * D + d] = O;
      if (d == 0) {
        a.part_md[prow * 2 + 0] = M;
        a.part_md[prow * 2 + 1] = Dn;
      }
    }
  }
  if (it.partial_slot >= 0 && a.fuse_merge) merge_if_last<D>(a, it, kvh, blockDim.x);
}

// Kernel selection (each translation unit provides its family). `rows` is the
// number of (query token, query head) rows one workgroup handles, over `hp`
// KV heads (2: a pair of KV heads per workgroup).
DecodeFn valu_decode_kernel(int kv_dtype, int head_dim, int group);
DecodeFn mfma_decode_kernel(int kv_dtype, int head_dim, int rows, int page_size, int hp);

}  // namespace pkd
