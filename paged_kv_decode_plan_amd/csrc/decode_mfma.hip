// MFMA split-KV paged decode kernel, for gfx950 (bf16 or e4m3 KV, bf16 q,
// head_dim 128, up to 16 query heads per KV head).
//
// What is computed ("FlashDecoding + FlashInfer — the decode-time attention
// story"): for one query token per request and each query head h, the softmax
// of scale * q.K over the request's KV tokens, applied to V; K/V rows are
// gathered through the page table (§"Paged attention (vLLM)"). A workgroup
// handles one work item (a run of one request's pages) for one KV head and the
// G query heads that share it and ends with either the output rows or partial
// (m, d, o) states (§"FlashDecoding — the split-KV trick"); within it the
// running (m, d, o) is updated tile by tile with the same rule.
//
// Both contractions run on v_mfma_f32_16x16x32_bf16 (A: 16 x 32, B: 32 x 16,
// fp32 C; lane l holds A row l%16 / B column l%16 for the k-slice
// 8*(l/16)..+8, and C rows 4*(l/16)..+4 of column l%16). The order in which a
// contraction visits its index is free as long as A and B agree; both
// products below use that freedom so that every operand comes straight from
// coalesced loads:
//
//   S = K . q^T   A = K (rows: 16 tokens), B = q^T (columns: query heads, zero
//                 beyond G), k = head_dim in four 32-wide steps. Lane l loads
//                 16 bytes of token l%16; the four lanes of a token read 64
//                 contiguous bytes per instruction.
//   O = P . V     A = P (rows: heads, k: 32 tokens), B = V (k: tokens,
//                 columns: dims). Lane l loads 16-byte chunk l%16 of a V row
//                 (16 lanes read one whole row), so it holds dims
//                 8*(l%16)..+8 of eight tokens; MFMA number nc (0..7) takes
//                 element nc of each, i.e. output column j is dim 8*j + nc.
//                 The eight tokens of lane l are exactly the eight scores
//                 that lane holds in the C layout of S, so P needs no lane
//                 exchange: k-slot e of quarter q is token 4q+e (e < 4) or
//                 16+4q+(e-4) (e >= 4) of the 32-token tile.
//
// P is fed to the bf16 MFMA as a hi + lo pair of bf16 values (two MFMAs),
// which keeps its 16 significant bits; V is exact in bf16 (e4m3 widens to
// bf16 exactly and its per-page scale is folded into P), and K.q products are
// exact with fp32 accumulation.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernel_common.h"

namespace pkd {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

constexpr int kD = 128;
constexpr int kTile = 32;  // tokens per wavefront tile

__device__ inline f32x4_t mfma(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Pack the low (sel_hi = false) or high 16-bit halves of two words: lo of the
// result from `a`, hi from `b`.
__device__ inline uint32_t pack_halves(uint32_t a, uint32_t b, bool sel_hi) {
  return __builtin_amdgcn_perm(b, a, sel_hi ? 0x07060302u : 0x05040100u);
}

__device__ inline bf16x8_t as_bf16x8(const u32x4_t& v) { return __builtin_bit_cast(bf16x8_t, v); }

// Two e4m3 bytes (half `hi` of a word) -> two bf16 (exact).
__device__ inline uint32_t e4m3x2_to_bf16x2(uint32_t w, bool hi) {
  return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(int(w), 1.0f, true))
            : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(int(w), 1.0f, false));
}

// Token (within a 32-token tile) that k-slot e of lane quarter q stands for in
// the P.V product; equal to the token of the lane's e-th score in the C layout
// of S (two 16-token groups, rows 4q..4q+3 of each).
__device__ inline int pv_token(int q, int e) { return e < 4 ? 4 * q + e : 16 + 4 * q + (e - 4); }

template <int KV>
struct Loads;

template <>
struct Loads<kBF16> {
  u32x4_t k[2][4];  // [token group][dc]: 8 dims of token 16*tg + l%16
  u32x4_t v[8];     // [e]: dims 8*(l%16)..+8 of token pv_token(q, e)
  static constexpr int kElem = 2;
};

template <>
struct Loads<kE4M3> {
  u32x4_t k[2][2];  // [token group][h]: 16 dims, 64 contiguous bytes per token and instruction
  uint2 v[8];       // [e]: dims 8*(l%16)..+8 of token pv_token(q, e)
  static constexpr int kElem = 1;
};

// The head_dim index visited by QK k-slot (dc, q, e): bf16 lanes load 8 dims at
// chunk 4*dc + q; e4m3 lanes load 16 dims at chunk 4*h + q and split them
// into dc = 2h (first 8) and dc = 2h + 1 (last 8).
template <int KV>
__device__ inline int qk_dim(int dc, int q, int e) {
  if constexpr (KV == kBF16)
    return 8 * (4 * dc + q) + e;
  else
    return 16 * (4 * (dc >> 1) + q) + 8 * (dc & 1) + e;
}

template <int KV, int G, bool PAGE16>
__global__ __launch_bounds__(kThreads) void decode_mfma_kernel(KernelArgs a) {
  static_assert(G >= 1 && G <= 16, "at most 16 query heads per KV head");
  __shared__ WaveStates<G, kD> st;

  const int kvh = blockIdx.x % a.num_kv_heads;
  const DeviceItem it = a.items[blockIdx.x / a.num_kv_heads];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int q4 = lane >> 4;  // lane quarter
  const int j = lane & 15;   // row/column index inside the 16x16 tiles
  const int log2p = a.page_size_log2;
  const int pmask = (1 << log2p) - 1;

  // q^T as the B operand of S = K.q^T: column j = query head kvh*G + j.
  bf16x8_t qb[4];
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (int64_t(it.request) * a.num_qo_heads + int64_t(kvh) * G + j) * kD;
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) {
      u32x4_t w = {0u, 0u, 0u, 0u};
      if (j < G) {
        w = *reinterpret_cast<const u32x4_t*>(qp + qk_dim<KV>(dc, q4, 0));
      }
      qb[dc] = as_bf16x8(w);
    }
  }

  f32x4_t acc[8];
#pragma unroll
  for (int nc = 0; nc < 8; ++nc) acc[nc] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // head j, log2 units, uniform over quarters
  float d_run = 0.f;        // head j, this lane's tokens

  const char* kbase = static_cast<const char*>(a.k);
  const char* vbase = static_cast<const char*>(a.v);
  constexpr int kElem = Loads<KV>::kElem;
  const int64_t head_off = int64_t(kvh) * a.head_stride;
  const int32_t* page_ids = a.indices + it.page_begin;
  const int kv_len = it.kv_len;

  for (int t0 = wave * kTile; t0 < kv_len; t0 += kWaves * kTile) {
    Loads<KV> ld;
    float kscale[2] = {1.f, 1.f}, vscale[2] = {1.f, 1.f};
    // ---- page lookups and loads
    int64_t gpage[2] = {0, 0};
    if constexpr (PAGE16) {
      // Pages of at least 16 tokens: each 16-token group lies in one page.
#pragma unroll
      for (int tg = 0; tg < 2; ++tg) {
        const int tt = t0 + 16 * tg;
        if (tt < kv_len) {
          gpage[tg] = page_ids[tt >> log2p];
          if constexpr (KV == kE4M3) {
            kscale[tg] = a.k_scale[gpage[tg] * a.num_kv_heads + kvh];
            vscale[tg] = a.v_scale[gpage[tg] * a.num_kv_heads + kvh];
          }
        }
      }
    }
#pragma unroll
    for (int tg = 0; tg < 2; ++tg) {
      const int t = t0 + 16 * tg + j;
      const bool ok = t < kv_len;
      int64_t page = gpage[tg];
      if constexpr (!PAGE16) page = ok ? page_ids[t >> log2p] : 0;
      const int64_t row = page * a.page_stride + int64_t(t & pmask) * a.token_stride + head_off;
      if constexpr (KV == kBF16) {
#pragma unroll
        for (int dc = 0; dc < 4; ++dc)
          ld.k[tg][dc] = ok ? *reinterpret_cast<const u32x4_t*>(
                                  kbase + (row + qk_dim<KV>(dc, q4, 0)) * kElem)
                            : u32x4_t{0u, 0u, 0u, 0u};
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h)
          ld.k[tg][h] = ok ? *reinterpret_cast<const u32x4_t*>(
                                 kbase + (row + qk_dim<KV>(2 * h, q4, 0)) * kElem)
                           : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int tau = pv_token(q4, e);
      const int t = t0 + tau;
      const bool ok = t < kv_len;
      int64_t page = gpage[tau >> 4];
      if constexpr (!PAGE16) page = ok ? page_ids[t >> log2p] : 0;
      const int64_t off =
          (page * a.page_stride + int64_t(t & pmask) * a.token_stride + head_off + 8 * j) * kElem;
      if constexpr (KV == kBF16)
        ld.v[e] = ok ? *reinterpret_cast<const u32x4_t*>(vbase + off) : u32x4_t{0u, 0u, 0u, 0u};
      else
        ld.v[e] = ok ? *reinterpret_cast<const uint2*>(vbase + off) : uint2{0u, 0u};
    }

    // ---- S = K . q^T for the two 16-token groups
    f32x4_t s[2];
#pragma unroll
    for (int tg = 0; tg < 2; ++tg) {
      f32x4_t c = {0.f, 0.f, 0.f, 0.f};
      if constexpr (KV == kBF16) {
#pragma unroll
        for (int dc = 0; dc < 4; ++dc) c = mfma(as_bf16x8(ld.k[tg][dc]), qb[dc], c);
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const u32x4_t w = ld.k[tg][h];
          u32x4_t lo, hi;  // dims 0..7 and 8..15 of the 16 loaded
          lo[0] = e4m3x2_to_bf16x2(w[0], false);
          lo[1] = e4m3x2_to_bf16x2(w[0], true);
          lo[2] = e4m3x2_to_bf16x2(w[1], false);
          lo[3] = e4m3x2_to_bf16x2(w[1], true);
          hi[0] = e4m3x2_to_bf16x2(w[2], false);
          hi[1] = e4m3x2_to_bf16x2(w[2], true);
          hi[2] = e4m3x2_to_bf16x2(w[3], false);
          hi[3] = e4m3x2_to_bf16x2(w[3], true);
          c = mfma(as_bf16x8(lo), qb[2 * h], c);
          c = mfma(as_bf16x8(hi), qb[2 * h + 1], c);
        }
      }
      s[tg] = c;
    }

    // ---- scale, mask and the tile max of head j
    float sc[8];
    float mt = -INFINITY;
#pragma unroll
    for (int tg = 0; tg < 2; ++tg) {
      float ks = a.sm_scale_log2;
      if constexpr (KV == kE4M3 && PAGE16) ks *= kscale[tg];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + 16 * tg + 4 * q4 + r;
        float kr = ks;
        if constexpr (KV == kE4M3 && !PAGE16) {
          kr = t < kv_len ? ks * a.k_scale[int64_t(page_ids[t >> log2p]) * a.num_kv_heads + kvh]
                          : ks;
        }
        const float v = t < kv_len ? s[tg][r] * kr : -INFINITY;
        sc[4 * tg + r] = v;
        mt = fmaxf(mt, v);
      }
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);  // finite: the tile holds a valid token
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;

    // ---- P (hi + lo bf16) in k-slot order: slot e <-> score sc[e]
    float p[8];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = exp2f(sc[e] - m_new);
      psum += p[e];
    }
    d_run = d_run * alpha + psum;
    if constexpr (KV == kE4M3) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float vs;
        if constexpr (PAGE16) {
          vs = vscale[e >> 2];
        } else {
          const int t = t0 + pv_token(q4, e);
          vs = t < kv_len ? a.v_scale[int64_t(page_ids[t >> log2p]) * a.num_kv_heads + kvh] : 0.f;
        }
        p[e] *= vs;
      }
    }
    bf16x8_t p_hi, p_lo;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const f32x2_t pp = {p[e], p[e + 1]};
      const bf16x2_t h = __builtin_convertvector(pp, bf16x2_t);
      const f32x2_t hf = __builtin_convertvector(h, f32x2_t);
      const f32x2_t rest = pp - hf;
      const bf16x2_t l = __builtin_convertvector(rest, bf16x2_t);
      p_hi[e] = h[0];
      p_hi[e + 1] = h[1];
      p_lo[e] = l[0];
      p_lo[e + 1] = l[1];
    }

    // ---- rescale O rows (heads 4*q4 + r) when any running max moved
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(alpha, 4 * q4 + r, 64);
#pragma unroll
        for (int nc = 0; nc < 8; ++nc) acc[nc][r] *= ar;
      }
    }

    // ---- O += P . V, column j of MFMA nc is dim 8*j + nc
#pragma unroll
    for (int nc = 0; nc < 8; ++nc) {
      u32x4_t vb;
      if constexpr (KV == kBF16) {
        const int w = nc >> 1;
        const bool hi = nc & 1;
#pragma unroll
        for (int pr = 0; pr < 4; ++pr)
          vb[pr] = pack_halves(ld.v[2 * pr][w], ld.v[2 * pr + 1][w], hi);
      } else {
        const int w = nc >> 2;          // word of the 8 loaded bytes
        const bool hiw = (nc >> 1) & 1;  // which byte pair in the word
        const bool hib = nc & 1;         // which byte of the pair
#pragma unroll
        for (int pr = 0; pr < 4; ++pr) {
          const uint32_t x0 = e4m3x2_to_bf16x2(w ? ld.v[2 * pr].y : ld.v[2 * pr].x, hiw);
          const uint32_t x1 = e4m3x2_to_bf16x2(w ? ld.v[2 * pr + 1].y : ld.v[2 * pr + 1].x, hiw);
          vb[pr] = pack_halves(x0, x1, hib);
        }
      }
      const bf16x8_t vbb = as_bf16x8(vb);
      acc[nc] = mfma(p_hi, vbb, acc[nc]);
      acc[nc] = mfma(p_lo, vbb, acc[nc]);
    }
  }

  // ---- per-wavefront state -> shared memory
  d_run += __shfl_xor(d_run, 16, 64);
  d_run += __shfl_xor(d_run, 32, 64);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * q4 + r;
    if (h < G) {
#pragma unroll
      for (int nc = 0; nc < 8; ++nc) st.o[wave][h][8 * j + nc] = acc[nc][r];
    }
  }
  if (q4 == 0 && j < G) {
    st.m[wave][j] = m_run;
    st.d[wave][j] = d_run;
  }
  __syncthreads();
  finish_workgroup<G, kD>(st, a, it, kvh);
}

template <int KV, bool P16>
DecodeFn pick_group(int g) {
  switch (g) {
    case 1: return decode_mfma_kernel<KV, 1, P16>;
    case 2: return decode_mfma_kernel<KV, 2, P16>;
    case 4: return decode_mfma_kernel<KV, 4, P16>;
    case 8: return decode_mfma_kernel<KV, 8, P16>;
    case 16: return decode_mfma_kernel<KV, 16, P16>;
    default: return nullptr;
  }
}

}  // namespace

DecodeFn mfma_decode_kernel(int kv_dtype, int head_dim, int group, int page_size) {
  if (head_dim != kD) return nullptr;
  const bool p16 = page_size >= 16;
  switch (kv_dtype) {
    case kBF16: return p16 ? pick_group<kBF16, true>(group) : pick_group<kBF16, false>(group);
    case kE4M3: return p16 ? pick_group<kE4M3, true>(group) : pick_group<kE4M3, false>(group);
    default: return nullptr;
  }
}

}  // namespace pkd
