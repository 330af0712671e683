// VALU split-KV paged decode kernel, for gfx950.
//
// What is computed ("FlashDecoding + FlashInfer — the decode-time attention
// story"): for one query token per request and each query head, the softmax of
// scale * q.K over the request's KV tokens, applied to V, with K/V rows
// gathered through the page table (§"Paged attention (vLLM)"). A workgroup
// handles one work item (a run of one request's pages) for one KV head and the
// G query heads that share it, producing the final output row or a partial
// (m, d, o) state (§"FlashDecoding — the split-KV trick").
//
// This is the vector-ALU kernel, used where the MFMA kernel does not apply
// (fp32 KV or queries, head_dim 64). Layout inside a workgroup (4 wavefronts):
//   * one K or V row is spread over LPR lanes, VEC elements (16 bytes, 8 for
//     e4m3) per lane, so one wavefront reads ROWS = 64 / LPR tokens per load;
//   * a wavefront processes tiles of ROWS * U consecutive tokens, wavefront w
//     taking tiles w, w + 4, ...; every tile's loads are issued before any of
//     its arithmetic;
//   * the G partial dot products of a lane are reduced across its row with a
//     reduce-scatter (each exchange halves the list of heads a lane carries),
//     so each lane finishes the score of one query head for its row's token
//     and exp() runs once per (token, head);
//   * the running max is per head and uniform across the wavefront; d and o
//     are per-lane partial sums, reduced across rows and wavefronts at the end.
// Scores are kept in log2 units (scale * log2(e) folded into one multiply).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernel_common.h"

namespace pkd {

namespace {

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

  __shared__ WaveStates<G, D> st;

  int item_idx, kvh;
  decode_block(a.num_kv_heads, a.xcd_group, &item_idx, &kvh);
  if (item_idx >= launch_items(a)) return;  // grid padding; no barrier passed yet
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
    const int64_t qbase = (int64_t(it.q_row) * a.num_qo_heads + int64_t(kvh) * G) * D + j * VEC;
#pragma unroll
    for (int p = 0; p < G; ++p) {
      const int h = p ^ own;
      const int64_t off = qbase + int64_t(h) * D;
      if (a.q_kind == kQBF16) {
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
      for (int e = 0; e < VEC; ++e) st.o[wave][h][j * VEC + e] = o[h][e];
    if ((j & ((LPR / G) - 1)) == 0) {
      st.m[wave][own] = m_run;
      st.d[wave][own] = d_run;
    }
  }
  __syncthreads();
  finish_workgroup<G, D>(st, a, it, kvh);
}


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

DecodeFn pick_kv(int kv, int d, int g) {
  switch (kv) {
    case kF32: return pick_dim<kF32>(d, g);
    case kBF16: return pick_dim<kBF16>(d, g);
    case kE4M3: return pick_dim<kE4M3>(d, g);
    default: return nullptr;
  }
}

}  // namespace

DecodeFn valu_decode_kernel(int kv_dtype, int head_dim, int group) {
  return pick_kv(kv_dtype, head_dim, group);
}

}  // namespace pkd
