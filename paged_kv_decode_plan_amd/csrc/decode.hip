// Split-KV paged decode attention and the partial-state merge, for gfx950.
//
// What is computed ("FlashDecoding + FlashInfer — the decode-time attention
// story"): for one query token per request and each query head h, the softmax
// of scale * q.K over the request's KV tokens, applied to V. K/V rows are
// gathered through the page table (§"Paged attention (vLLM)"). Each workgroup
// handles one work item (a run of one request's pages) for one KV head and the
// `G` query heads that share it, producing either the final output or a
// partial (m, d, o) state (§"FlashDecoding — the split-KV trick"); a second
// kernel merges the partials of split requests with the online-softmax rule.
//
// Layout of the work inside a workgroup (4 wavefronts of 64 lanes):
//   * one K or V row (head_dim elements) is spread over LPR lanes, VEC
//     elements (16 bytes, 8 for e4m3) per lane, so one wavefront reads
//     ROWS = 64 / LPR tokens per 128-bit load instruction;
//   * a wavefront processes tiles of ROWS * U consecutive tokens, wavefront w
//     taking tiles w, w + 4, w + 8, ...; every tile's K and V loads are issued
//     before any of its arithmetic;
//   * the G partial dot products of a lane are reduced across its row with a
//     reduce-scatter (each exchange halves the list of heads a lane carries),
//     so each lane ends up owning the full score of one query head for its
//     row's token; exp() is evaluated once per (token, head);
//   * the running max m is kept per head and uniform across the wavefront;
//     d and o are per-lane partial sums, reduced across rows and wavefronts
//     once at the end with the same merge rule.
// Scores are kept in log2 units (scale * log2(e) folded into one multiply)
// so exp() is a single exp2 instruction.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "launch.h"

namespace pkd {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

template <int KV>
struct Kv;
template <>
struct Kv<kF32> {
  static constexpr int kVec = 4;  // elements per lane per load (16 bytes)
  using Raw = uint4;
  __device__ static inline void unpack(const Raw& r, float (&f)[kVec]) {
    f[0] = __uint_as_float(r.x);
    f[1] = __uint_as_float(r.y);
    f[2] = __uint_as_float(r.z);
    f[3] = __uint_as_float(r.w);
  }
};
template <>
struct Kv<kBF16> {
  static constexpr int kVec = 8;  // 16 bytes
  using Raw = uint4;
  __device__ static inline void unpack(const Raw& r, float (&f)[kVec]) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <>
struct Kv<kE4M3> {
  static constexpr int kVec = 8;  // 8 bytes
  using Raw = uint2;
  __device__ static inline void unpack(const Raw& r, float (&f)[kVec]) {
    const uint32_t w[2] = {r.x, r.y};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(int(w[i]), false);
      auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(int(w[i]), true);
      f[4 * i + 0] = lo[0];
      f[4 * i + 1] = lo[1];
      f[4 * i + 2] = hi[0];
      f[4 * i + 3] = hi[1];
    }
  }
};

__device__ inline float lane_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }
__device__ inline float lane_read(float v, int src) { return __shfl(v, src, 64); }

__device__ inline float bf16_bits_to_float(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

__device__ inline uint16_t float_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Reduce the G per-lane partial dot products across the LPR lanes of a row.
// On entry position p of lane j holds the partial for head p ^ own(j), with
// own(j) = j >> (log2(LPR) - log2(G)); on return the lane holds the full dot
// product of head own(j).
template <int LPR, int G>
__device__ inline float row_reduce_scatter(float (&v)[G], int j_unused) {
  constexpr int kLogL = ilog2(LPR);
  constexpr int kLogG = ilog2(G);
  static_assert(G <= LPR, "group larger than a row");
#pragma unroll
  for (int s = 0; s < kLogG; ++s) {
    const int half = G >> (s + 1);
    const int mask = 1 << (kLogL - 1 - s);
#pragma unroll
    for (int i = 0; i < half; ++i) v[i] += lane_xor(v[half + i], mask);
  }
  float x = v[0];
#pragma unroll
  for (int b = kLogL - kLogG - 1; b >= 0; --b) x += lane_xor(x, 1 << b);
  (void)j_unused;
  return x;
}

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
  const DeviceItem* items;
  float* part_o;
  float* part_md;
  int num_kv_heads;
  int num_qo_heads;
  int page_size_log2;
  float sm_scale_log2;
  int q_bf16;
  int out_bf16;
};

template <int KV, int D, int G>
__global__ __launch_bounds__(kThreads) void decode_kernel(KernelArgs a) {
  using T = Kv<KV>;
  constexpr int VEC = T::kVec;
  constexpr int LPR = D / VEC;          // lanes per K/V row
  constexpr int ROWS = 64 / LPR;        // tokens per wavefront per load
  constexpr int U = (KV == kE4M3) ? 8 : 4;  // loads in flight per lane per tile
  constexpr int TILE = ROWS * U;        // tokens per wavefront tile
  constexpr int kLogL = ilog2(LPR);
  constexpr int kLogG = ilog2(G);
  static_assert(LPR * ROWS == 64, "row layout");

  __shared__ float sm_o[kWaves][G][D];
  __shared__ float sm_m[kWaves][G];
  __shared__ float sm_d[kWaves][G];

  const int kvh = blockIdx.x % a.num_kv_heads;
  const int item_idx = blockIdx.x / a.num_kv_heads;
  const DeviceItem it = a.items[item_idx];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row = lane / LPR;
  const int j = lane % LPR;
  const int own = j >> (kLogL - kLogG);  // head whose score this lane finishes
  const int P = 1 << a.page_size_log2;

  // q for this lane's VEC dims, head order permuted per lane (see row_reduce_scatter).
  float qr[G][VEC];
  {
    const int64_t qbase = (int64_t(it.request) * a.num_qo_heads + int64_t(kvh) * G) * D + j * VEC;
#pragma unroll
    for (int p = 0; p < G; ++p) {
      const int h = p ^ own;
      const int64_t off = qbase + int64_t(h) * D;
      if (a.q_bf16) {
        const uint16_t* qp = static_cast<const uint16_t*>(a.q) + off;
#pragma unroll
        for (int e = 0; e < VEC; ++e) qr[p][e] = bf16_bits_to_float(qp[e]);
      } else {
        const float* qp = static_cast<const float*>(a.q) + off;
#pragma unroll
        for (int e = 0; e < VEC; ++e) qr[p][e] = qp[e];
      }
    }
  }

  float o[G][VEC];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < VEC; ++e) o[h][e] = 0.f;
  float m_run = -INFINITY;  // log2 units, head `own`, uniform over rows
  float d_run = 0.f;        // this row's share, head `own`

  const char* kbase = static_cast<const char*>(a.k);
  const char* vbase = static_cast<const char*>(a.v);
  constexpr int kElem = (KV == kF32) ? 4 : (KV == kBF16 ? 2 : 1);
  const int64_t lane_off = int64_t(kvh) * a.head_stride + j * VEC;
  const int32_t* page_ids = a.indices + it.page_begin;

  for (int t0 = wave * TILE; t0 < it.kv_len; t0 += kWaves * TILE) {
    typename T::Raw kraw[U], vraw[U];
    float ks[U], vs[U];
    bool valid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + u * ROWS + row;
      valid[u] = t < it.kv_len;
      ks[u] = 1.f;
      vs[u] = 1.f;
      if (valid[u]) {
        const int64_t page = page_ids[t >> a.page_size_log2];
        const int slot = t & (P - 1);
        const int64_t off = page * a.page_stride + int64_t(slot) * a.token_stride + lane_off;
        kraw[u] = *reinterpret_cast<const typename T::Raw*>(kbase + off * kElem);
        vraw[u] = *reinterpret_cast<const typename T::Raw*>(vbase + off * kElem);
        if constexpr (KV == kE4M3) {
          ks[u] = a.k_scale[page * a.num_kv_heads + kvh];
          vs[u] = a.v_scale[page * a.num_kv_heads + kvh];
        }
      } else {
        kraw[u] = typename T::Raw{};
        vraw[u] = typename T::Raw{};
      }
    }

    float s[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[VEC];
      T::unpack(kraw[u], kf);
      float part[G];
#pragma unroll
      for (int p = 0; p < G; ++p) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc = fmaf(qr[p][e], kf[e], acc);
        part[p] = acc;
      }
      const float dot = row_reduce_scatter<LPR, G>(part, j);
      s[u] = valid[u] ? dot * ks[u] * a.sm_scale_log2 : -INFINITY;
    }

    float mt = s[0];
#pragma unroll
    for (int u = 1; u < U; ++u) mt = fmaxf(mt, s[u]);
#pragma unroll
    for (int b = LPR; b < 64; b <<= 1) mt = fmaxf(mt, lane_xor(mt, b));
    const float m_new = fmaxf(m_run, mt);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;

    float pv[U];
    float psum = 0.f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float p = exp2f(s[u] - m_new);
      psum += p;
      pv[u] = p * vs[u];
    }
    d_run = d_run * alpha + psum;

    const int row_base = row * LPR;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float ah = lane_read(alpha, row_base + (h << (kLogL - kLogG)));
#pragma unroll
      for (int e = 0; e < VEC; ++e) o[h][e] *= ah;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[VEC];
      T::unpack(vraw[u], vf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float ph = lane_read(pv[u], row_base + (h << (kLogL - kLogG)));
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[h][e] = fmaf(ph, vf[e], o[h][e]);
      }
    }
  }

  // Reduce d and o over the rows of the wavefront (m is already uniform).
#pragma unroll
  for (int b = LPR; b < 64; b <<= 1) {
    d_run += lane_xor(d_run, b);
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < VEC; ++e) o[h][e] += lane_xor(o[h][e], b);
  }
  if (row == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < VEC; ++e) sm_o[wave][h][j * VEC + e] = o[h][e];
    if ((j & ((LPR / G) - 1)) == 0) {
      sm_m[wave][own] = m_run;
      sm_d[wave][own] = d_run;
    }
  }
  __syncthreads();

  // Merge the wavefronts' states and write the output or the partial state.
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D;
    const int d = idx % D;
    float M = sm_m[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm_m[w][h]);
    float O = 0.f, Dn = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float sc = exp2f(sm_m[w][h] - M);
      O = fmaf(sm_o[w][h][d], sc, O);
      Dn = fmaf(sm_d[w][h], sc, Dn);
    }
    const int hq = kvh * G + h;
    const int64_t row_idx = int64_t(it.request) * a.num_qo_heads + hq;
    if (it.partial_slot < 0) {
      const float val = O / Dn;
      if (a.out_bf16)
        static_cast<uint16_t*>(a.out)[row_idx * D + d] = float_to_bf16_rne(val);
      else
        static_cast<float*>(a.out)[row_idx * D + d] = val;
      if (a.lse && d == 0) a.lse[row_idx] = (M + log2f(Dn)) * 0.69314718055994530942f;
    } else {
      const int64_t prow = int64_t(it.partial_slot) * a.num_qo_heads + hq;
      a.part_o[prow * D + d] = O;
      if (d == 0) {
        a.part_md[prow * 2 + 0] = M;
        a.part_md[prow * 2 + 1] = Dn;
      }
    }
  }
}

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

// One workgroup per (split request, query head); one thread per output
// element. Folds the request's partial states with the merge rule and
// normalises: out = o / d, lse = m + ln d.
template <int D>
__global__ __launch_bounds__(D) void merge_kernel(MergeArgs a) {
  const int hq = blockIdx.x % a.num_qo_heads;
  const int j = blockIdx.x / a.num_qo_heads;
  const int r = a.split_requests[j];
  const int b = a.merge_indptr[r];
  const int e = a.merge_indptr[r + 1];
  const int d = threadIdx.x;
  float M = -INFINITY;
  for (int i = b; i < e; ++i) M = fmaxf(M, a.part_md[(int64_t(i) * a.num_qo_heads + hq) * 2]);
  float O = 0.f, Dn = 0.f;
  for (int i = b; i < e; ++i) {
    const int64_t prow = int64_t(i) * a.num_qo_heads + hq;
    const float sc = exp2f(a.part_md[prow * 2] - M);
    Dn = fmaf(a.part_md[prow * 2 + 1], sc, Dn);
    O = fmaf(a.part_o[prow * D + d], sc, O);
  }
  const int64_t row_idx = int64_t(r) * a.num_qo_heads + hq;
  const float val = O / Dn;
  if (a.out_bf16)
    static_cast<uint16_t*>(a.out)[row_idx * D + d] = float_to_bf16_rne(val);
  else
    static_cast<float*>(a.out)[row_idx * D + d] = val;
  if (a.lse && d == 0) a.lse[row_idx] = (M + log2f(Dn)) * 0.69314718055994530942f;
}

using DecodeFn = void (*)(KernelArgs);

template <int KV, int D>
DecodeFn pick_group(int g) {
  switch (g) {
    case 1: return decode_kernel<KV, D, 1>;
    case 2: return decode_kernel<KV, D, 2>;
    case 4: return decode_kernel<KV, D, 4>;
    case 8: return decode_kernel<KV, D, 8>;
    default: return nullptr;
  }
}

template <int KV>
DecodeFn pick_dim(int d, int g) {
  switch (d) {
    case 64: return pick_group<KV, 64>(g);
    case 128: return pick_group<KV, 128>(g);
    default: return nullptr;
  }
}

DecodeFn pick(int kv, int d, int g) {
  switch (kv) {
    case kF32: return pick_dim<kF32>(d, g);
    case kBF16: return pick_dim<kBF16>(d, g);
    case kE4M3: return pick_dim<kE4M3>(d, g);
    default: return nullptr;
  }
}

}  // namespace

bool decode_supported(int kv_dtype, int head_dim, int group) {
  return pick(kv_dtype, head_dim, group) != nullptr;
}

hipError_t launch_decode(const DecodeLaunch& L, hipStream_t stream) {
  DecodeFn fn = pick(L.kv_dtype, L.head_dim, L.group);
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
  a.items = L.items;
  a.part_o = L.part_o;
  a.part_md = L.part_md;
  a.num_kv_heads = L.num_kv_heads;
  a.num_qo_heads = L.num_qo_heads;
  a.page_size_log2 = L.page_size_log2;
  a.sm_scale_log2 = L.sm_scale_log2;
  a.q_bf16 = L.q_bf16;
  a.out_bf16 = L.out_bf16;
  const unsigned grid = unsigned(L.num_items) * unsigned(L.num_kv_heads);
  hipLaunchKernelGGL(fn, dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

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
  if (L.head_dim == 64)
    hipLaunchKernelGGL(merge_kernel<64>, dim3(grid), dim3(64), 0, stream, a);
  else if (L.head_dim == 128)
    hipLaunchKernelGGL(merge_kernel<128>, dim3(grid), dim3(128), 0, stream, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t decode_occupancy(int kv_dtype, int head_dim, int group, int* wgs_per_cu) {
  DecodeFn fn = pick(kv_dtype, head_dim, group);
  if (!fn) return hipErrorInvalidValue;
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(wgs_per_cu, fn, kThreads, 0);
}

}  // namespace pkd
