// MFMA split-KV paged decode kernel, for gfx950 (bf16, e4m3 or e2m1 KV with
// bf16 q, fp16 KV with fp16 q; head_dim 128, up to 32 query rows per
// workgroup in one or two groups of 16 MFMA columns).
//
// What is computed ("FlashDecoding + FlashInfer — the decode-time attention
// story"): for each query token of a request and each query head h, the
// softmax of scale * q.K over the request's KV tokens, applied to V; K/V rows
// are gathered through the page table (§"Paged attention (vLLM)"). A
// workgroup handles one work item (a run of one request's pages, for a block
// of that request's query tokens) for one KV head and ends with either the
// output rows or partial (m, d, o) states (§"FlashDecoding — the split-KV
// trick"); within it the running (m, d, o) is updated tile by tile with the
// same rule. Its G rows are (query token i, query head hh of the group) with
// row = i * group + hh: the group's heads for one token per request, or, with
// several new tokens per request (the ragged q rows of §"Ragged attention"),
// up to 32 / group tokens, token i seeing the first min(kv_len, visible + i)
// tokens of the item (causal within the new tokens). Rows 16..31 form a
// second group of MFMA columns that shares every K and V load.
//
// Both contractions run on MFMA: S = K.q^T on v_mfma_f32_16x16x32_bf16 and
// O = P.V on v_mfma_f32_16x16x16_bf16, or on the k = 32 form over two
// sub-tiles (lane l holds A row l%16 / B column l%16 for a k-slice chosen by
// l/16, and C rows 4*(l/16)..+4 of column l%16).
// The order in which a contraction visits its index is free as long as A and B
// agree; both products use that freedom so that every operand comes straight
// from coalesced loads. A wavefront works on 16-token tiles:
//
//   S = K . q^T   A = K (rows: the 16 tokens), B = q^T (columns: query heads,
//                 zero beyond G), k = head_dim in four 32-wide steps. Lane l
//                 loads 16 bytes of token l%16; the four lanes of a token read
//                 64 contiguous bytes per instruction.
//   O = P . V     A = P (rows: heads, k: the 16 tokens), B = V (k: tokens,
//                 columns: dims). Lane l loads 16-byte chunk l%16 of a V row
//                 (16 lanes read one whole row), so it holds dims
//                 8*(l%16)..+8 of four tokens; MFMA number nc (0..7) takes
//                 element nc of each, i.e. output column j is dim 8*j + nc.
//                 The four tokens of lane l (4*(l/16)..+4) are the four scores
//                 that lane holds in the C layout of S, so P needs no lane
//                 exchange.
//
// While one tile is computed the next one's loads are in flight (two register
// buffers), and page ids come from a per-wavefront block of 64 tiles' ids
// held one per lane and read with readlane, so neither waits inside the loop.
//
// P is fed to the bf16 MFMA as a hi + lo pair of bf16 values (two MFMAs),
// which keeps its 16 significant bits; V is exact in bf16 (e4m3 widens to
// bf16 exactly and its per-page scale is folded into P), and K.q products are
// exact with fp32 accumulation.
//
// FP4 E2M1 KV (64-byte rows, one fp32 scale per KV head and channel): a lane
// loads 16 bytes = 32 dims of its K row and 4 bytes = 8 dims of each of its
// four V rows. E2M1 widens to bf16 exactly; the K channel scales are folded
// into q (q * k_scale as a hi + lo bf16 pair, two MFMAs per k step) and the V
// channel scales multiply the finished O columns.
//
// Two KV heads per workgroup (HP = 2): a 64-byte e2m1 row is half a 128-byte
// cache line whose other half is the next KV head's row, and an e4m3 row is
// one line. Workgroups that each read one head's e2m1 rows reach only about
// 55% of HBM bandwidth on MI355X, and with one resident workgroup per CU the
// bytes a workgroup reads contiguously per token keep mattering up to 256
// (one bf16 row). So a workgroup may take an even-odd pair of KV heads, and a
// sub-tile's 16 S rows are 8 tokens x 2 heads (row rho is token rho % 8 of
// head rho / 8), so that each load instruction reads both heads' rows of a
// token side by side. The S columns are the pair's rows (2 * group query
// heads per token; two column groups when they exceed 16); a
// lane's four S values all belong to one head (quarter q4 / 2), and those
// whose head is not their column's are masked to -inf, so P.V over the 16
// rows sums each column's own head only. The MFMA work per head is unchanged.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernel_common.h"

namespace pkd {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4_t;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(4))) short i16x4_t;

constexpr int kD = 128;
constexpr int kSub = 16;        // tokens per MFMA sub-tile
constexpr float kSlack = 8.0f;  // log2 headroom of the lazy reference max

// Sub-tiles per wavefront tile: a tile should bring about 8 KiB of K and V
// per wavefront, so e4m3 (128-byte rows) takes two 16-token sub-tiles. The
// 4-bit forms, which run two or three workgroups per CU, take two (4 KiB):
// measured on MI355X, e2m1 447 -> 409 us and int4 452 -> 433 us per step
// against four sub-tiles (8 KiB), whose registers also made int4's third
// workgroup spill.
#ifndef PKD_E4M3_NSUB
#define PKD_E4M3_NSUB 2
#endif
#ifndef PKD_BF16_NSUB
#define PKD_BF16_NSUB 1
#endif
#ifndef PKD_E2M1_NSUB
#define PKD_E2M1_NSUB 2
#endif
template <int KV>
constexpr bool fp8() { return KV == kE4M3 || KV == kE4M3T; }
template <int KV>
constexpr bool nib4() { return KV == kE2M1 || KV == kI4; }  // 4-bit codes, two per byte
// 16-bit KV rows (bf16 or fp16): 256 bytes per row at head_dim 128.
template <int KV>
constexpr bool wide16() { return KV == kBF16 || KV == kF16; }
template <int KV>
constexpr int nsub() { return fp8<KV>() ? PKD_E4M3_NSUB : nib4<KV>() ? PKD_E2M1_NSUB : PKD_BF16_NSUB; }
// Byte offset of an element offset (e2m1: two elements per byte; offsets
// handed to this are even).
template <int KV>
__device__ inline int64_t kv_bytes(int64_t elems) {
  if constexpr (nib4<KV>())
    return elems >> 1;
  else
    return elems * (wide16<KV>() ? 2 : 1);
}
// 16-byte K loads per lane and sub-tile.
template <int KV>
constexpr int k_loads() { return wide16<KV>() ? 4 : fp8<KV>() ? 2 : 1; }
// q operands per lane: four k steps, and for e2m1 a hi and a lo half each.
template <int KV>
constexpr int q_ops() { return nib4<KV>() ? 8 : 4; }
// Tokens per sub-tile: 16, or 16 / HP when the 16 rows are HP KV heads' rows.
template <int HP>
constexpr int sub_tokens() { return kSub / HP; }
template <int HP>
constexpr int sub_tokens_log2() {
  static_assert(HP == 1 || HP == 2, "one or two KV heads per workgroup");
  return HP == 1 ? 4 : 3;
}
// Token (within the sub-tile) of S row 4*q4 + r, and the KV head (within the
// workgroup's HP) of the lane's rows 4*q4 .. 4*q4 + 3.
template <int HP>
__device__ inline int row_token(int q4, int r) { return ((4 * q4) & (sub_tokens<HP>() - 1)) + r; }
template <int HP>
__device__ inline int row_head(int q4) { return (4 * q4) >> sub_tokens_log2<HP>(); }
template <int KV, int HP>
constexpr int tile_tokens() { return sub_tokens<HP>() * nsub<KV>(); }

// k = 32 step of S = K.q^T on eight 16-bit values per lane: fp16 for fp16 KV
// (with fp16 q), bf16 for every other form (bf16 q).
template <int KV>
__device__ inline f32x4_t mfma(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  if constexpr (KV == kF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// k = 16 step of O = P.V; operands are four 16-bit bit patterns.
template <int KV>
__device__ inline f32x4_t mfma16(uint2 a, uint2 b, const f32x4_t& c) {
  if constexpr (KV == kF16)
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                 __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4_t, a),
                                                     __builtin_bit_cast(i16x4_t, b), c, 0, 0, 0);
}

// p (fp32) as a hi + lo pair of the MFMA's 16-bit type: hi = round(p),
// lo = round(p - hi); together they carry 16 (bf16) or 22 (fp16) bits.
template <int KV>
__device__ inline void split16(float p0, float p1, uint32_t& hi, uint32_t& lo) {
  const f32x2_t pp = {p0, p1};
  if constexpr (KV == kF16) {
    const f16x2_t h = __builtin_convertvector(pp, f16x2_t);
    const f16x2_t l = __builtin_convertvector(pp - __builtin_convertvector(h, f32x2_t), f16x2_t);
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, l);
  } else {
    const bf16x2_t h = __builtin_convertvector(pp, bf16x2_t);
    const bf16x2_t l = __builtin_convertvector(pp - __builtin_convertvector(h, f32x2_t), bf16x2_t);
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, l);
  }
}

// Pack the low (sel_hi = false) or high 16-bit halves of two words: lo of the
// result from `a`, hi from `b`.
__device__ inline uint32_t pack_halves(uint32_t a, uint32_t b, bool sel_hi) {
  return __builtin_amdgcn_perm(b, a, sel_hi ? 0x07060302u : 0x05040100u);
}


// Raw buffer loads: a wavefront-uniform descriptor (the tile's first row) plus
// a 32-bit lane offset and a wavefront-uniform offset, so a tile's loads need
// no per-lane 64-bit address arithmetic.
__device__ inline __amdgpu_buffer_rsrc_t tile_rsrc(const char* p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), short(0), 0x7fffffff, 0x00020000);
}
// Cache policy of the K and V loads. V rows are read whole (16 lanes x 16 B)
// and exactly once, so they are marked non-temporal (NT); K rows arrive in two
// 64-byte halves of each 128-byte line from consecutive instructions, which
// the default policy serves from one line fill, so K keeps it. (Measured on
// MI355X: this pair beat all-default and all-NT for bf16 and e4m3 alike.)
#ifndef PKD_K_CPOL
#define PKD_K_CPOL 0
#endif
#ifndef PKD_V_CPOL
#define PKD_V_CPOL 2
#endif
template <int CPOL>
__device__ inline u32x4_t bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, int(voff), int(soff), CPOL));
}
template <int CPOL>
__device__ inline uint2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, int(voff), int(soff), CPOL));
}
template <int CPOL>
__device__ inline uint32_t bload4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, int(voff), int(soff), CPOL);
}

// Two e4m3 bytes (half `hi` of a word) -> two bf16 (exact).
__device__ inline uint32_t e4m3x2_to_bf16x2(uint32_t w, bool hi) {
  return hi ? __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(int(w), 1.0f, true))
            : __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(int(w), 1.0f, false));
}

// Byte B of a word (two e2m1 codes, the low nibble first) -> two bf16 (exact).
template <int B>
__device__ inline uint32_t e2m1x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, B));
}
// Eight e2m1 codes (a word, element 0 in the low nibble) -> eight bf16.
__device__ inline u32x4_t e2m1x8_to_bf16x8(uint32_t w) {
  return u32x4_t{e2m1x2_to_bf16x2<0>(w), e2m1x2_to_bf16x2<1>(w), e2m1x2_to_bf16x2<2>(w),
                 e2m1x2_to_bf16x2<3>(w)};
}

// Eight int4 codes (a word, element 0 in the low nibble, two's complement)
// -> eight bf16 holding (code + 8) * 2^-9 exactly. XOR 8 turns code c into
// the unsigned k = c + 8 in [0, 15], and a byte 0x0k read as e4m3 is exactly
// k * 2^-9 (subnormals 0..7 and the first binade 8..15 continue one
// another), so the fp8 conversion widens it. The output visits the word's
// dims in the order 0, 2, 4, 6, 1, 3, 5, 7 (low nibbles, then high nibbles);
// the q operand takes the same order, and the +8 and 2^-9 are undone in the
// score (a per-row term) and in the output.
__device__ inline u32x4_t i4x8_to_bf16x8(uint32_t w) {
  const uint32_t x = w ^ 0x88888888u;
  const uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
  return u32x4_t{e4m3x2_to_bf16x2(lo, false), e4m3x2_to_bf16x2(lo, true),
                 e4m3x2_to_bf16x2(hi, false), e4m3x2_to_bf16x2(hi, true)};
}

template <int KV>
struct Loads;

template <>
struct Loads<kBF16> {
  u32x4_t k[4];  // [dc]: 8 dims of token l%16
  u32x4_t v[4];  // [e]: dims 8*(l%16)..+8 of token 4*(l/16) + e
};

template <>
struct Loads<kF16> : Loads<kBF16> {};

template <>
struct Loads<kE4M3> {
  u32x4_t k[2];  // [h]: 16 dims of token l%16, 64 contiguous bytes per token and instruction
  uint2 v[4];    // [e]: dims 8*(l%16)..+8 of token 4*(l/16) + e
};

// e4m3 with row-wise scales: the same bytes, plus the K and V scales of the
// four tokens 4*(l/16) + e whose scores (and P weights) this lane holds.
template <>
struct Loads<kE4M3T> {
  u32x4_t k[2];
  uint2 v[4];
  float ks[4];
  float vs[4];
};

// e2m1: 32 dims of token l%16 (word dc holds dims 8*dc..+8 of them), and
// dims 8*(l%16)..+8 of token 4*(l/16) + e.
template <>
struct Loads<kE2M1> {
  u32x4_t k[1];
  uint32_t v[4];
};

template <>
struct Loads<kI4> : Loads<kE2M1> {};

// The head_dim index visited by QK k-slot (dc, q, e): bf16 lanes load 8 dims at
// chunk 4*dc + q; e4m3 lanes load 16 dims at chunk 4*h + q and split them
// into dc = 2h (first 8) and dc = 2h + 1 (last 8); e2m1 lanes load dims
// 32*q..+32 and take 8 of them per step.
template <int KV>
__device__ inline int qk_dim(int dc, int q, int e) {
  if constexpr (wide16<KV>())
    return 8 * (4 * dc + q) + e;
  else if constexpr (nib4<KV>())
    return 32 * q + 8 * dc + e;
  else
    return 16 * (4 * (dc >> 1) + q) + 8 * (dc & 1) + e;
}

// Where a sub-tile lives: with pages of at least 16 tokens a sub-tile (16 or
// 8 tokens) lies in one page (sub-tiles start at multiples of their size
// and items at page boundaries), so it needs one page id (wavefront-uniform)
// and, for e4m3, the page's K and V scale of the lane's own KV head (the head
// of its S rows and V rows), picked once when the page id is read. A sub-tile
// wholly past the item's end is given the page of the item's last sub-tile
// (its loads repeat valid tokens and its weights are 0).
struct TilePages {
  int64_t page;
  float ks, vs;  // e4m3 per-page scales of this lane's KV head
};

struct Ctx {
  const char* kbase;
  const char* vbase;
  // The K and V rows of this workgroup's (first) KV head in page 0, slot 0,
  // and the page and token strides in bytes (a page spans less than 4 GiB,
  // which the library checks), for the 4-bit forms' tile bases.
  const char* kbase_h;
  const char* vbase_h;
  uint32_t page_bytes, token_bytes;
  const int32_t* page_ids;  // the item's slice of the page table
  const float* k_scale;     // row-wise e4m3 scales (kE4M3T only)
  const float* v_scale;
  int num_kv_heads, kvh;  // KV heads of the pool; this workgroup's (first) head
  int64_t page_stride, token_stride, head_stride, head_off;
  int log2p, pmask, kv_len, q4, j;
  // Head pairs: the head (0, 1) of this lane's S rows and V rows.
  int head_lane;
  // Byte offsets of this lane's first K and V load from the tile's first row
  // (the same for every tile when a tile lies in one page); the other loads
  // add 64 bytes (K) or one token row (V), both wavefront-uniform.
  uint32_t koff;
  uint32_t voff;
  int64_t vrow_bytes;
};

// Issue every K and V load of the sub-tile starting at token t0.
// Every lane issues every load on every path: a token past the end of the
// item reads the item's last token instead (its score is masked to -inf and
// its P weight is 0, so it never contributes), which keeps the number of loads
// in flight the same on all paths and lets the next tile's loads overlap this
// tile's math.
template <int KV, bool PAGE16, bool FULL, int HP>
__device__ inline void issue_sub(Loads<KV>& ld, const Ctx& c, int t0, const TilePages& tp) {
  static_assert(HP == 1 || PAGE16, "head pairs: pages >= 16");
  constexpr int STL = sub_tokens_log2<HP>();
  const int last = c.kv_len - 1;
  constexpr int NK = k_loads<KV>();
  if constexpr (PAGE16) {
    // One page per sub-tile: a wavefront-uniform base plus lane offsets. A
    // sub-tile past the end loads from the last sub-tile's rows (tp.page is
    // that sub-tile's page).
    const int tb = FULL ? t0 : min(t0, last & ~(sub_tokens<HP>() - 1));
    __amdgpu_buffer_rsrc_t kr, vr;
    if constexpr (nib4<KV>()) {
      // 32-bit byte offsets within the page on top of the KV head's row in
      // page 0: fewer live scalar registers, which the 4-bit head-pair
      // instances need (their tile loop otherwise reloads spilled ones)
      const uint64_t base = uint64_t(uint32_t(tp.page)) * c.page_bytes +
                            uint32_t(tb & c.pmask) * c.token_bytes;
      kr = tile_rsrc(c.kbase_h + base);
      vr = tile_rsrc(c.vbase_h + base);
    } else {
      // (the same addresses from 64-bit element offsets: with the form above
      // the row-wise e4m3 kernel ran 10 % slower on MI355X, the others alike)
      const int64_t base = kv_bytes<KV>(tp.page * c.page_stride +
                                        int64_t(tb & c.pmask) * c.token_stride + c.head_off);
      kr = tile_rsrc(c.kbase + base);
      vr = tile_rsrc(c.vbase + base);
    }
    uint32_t koff = c.koff;
    if constexpr (!FULL) {
      if constexpr (HP > 1) {  // row j: token j % (16 / HP) of head j / (16 / HP)
        const int tk = min(t0 + (c.j & ((1 << STL) - 1)), last) - tb;
        koff = uint32_t(kv_bytes<KV>(int64_t(tk) * c.token_stride + (c.j >> STL) * c.head_stride +
                                     qk_dim<KV>(0, c.q4, 0)));
      } else {
        const int tk = min(t0 + c.j, last) - tb;
        koff = uint32_t(kv_bytes<KV>(int64_t(tk) * c.token_stride + qk_dim<KV>(0, c.q4, 0)));
      }
    }
#pragma unroll
    for (int x = 0; x < NK; ++x) ld.k[x] = bload16<PKD_K_CPOL>(kr, koff + 64 * x, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t voff, soff;
      if constexpr (FULL) {
        voff = c.voff;
        soff = uint32_t(e * c.vrow_bytes);
      } else {
        if constexpr (HP > 1) {  // rows 4*q4 + e of head head_lane
          const int tv = min(t0 + row_token<HP>(c.q4, e), last) - tb;
          voff = uint32_t(kv_bytes<KV>(int64_t(tv) * c.token_stride + c.head_lane * c.head_stride +
                                       8 * c.j));
        } else {
          const int tv = min(t0 + 4 * c.q4 + e, last) - tb;
          voff = uint32_t(kv_bytes<KV>(int64_t(tv) * c.token_stride + 8 * c.j));
        }
        soff = 0;
      }
      if constexpr (wide16<KV>())
        ld.v[e] = bload16<PKD_V_CPOL>(vr, voff, soff);
      else if constexpr (nib4<KV>())
        ld.v[e] = bload4<PKD_V_CPOL>(vr, voff, soff);
      else
        ld.v[e] = bload8<PKD_V_CPOL>(vr, voff, soff);
    }
  } else {
    {
      const int t = FULL ? t0 + c.j : min(t0 + c.j, last);
      const int64_t page = c.page_ids[t >> c.log2p];
      const int64_t row = page * c.page_stride + int64_t(t & c.pmask) * c.token_stride + c.head_off;
#pragma unroll
      for (int x = 0; x < NK; ++x) {
        const int dim = wide16<KV>() ? qk_dim<KV>(x, c.q4, 0) : qk_dim<KV>(2 * x, c.q4, 0);
        ld.k[x] = *reinterpret_cast<const u32x4_t*>(c.kbase + kv_bytes<KV>(row + dim));
      }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int t = FULL ? t0 + 4 * c.q4 + e : min(t0 + 4 * c.q4 + e, last);
      const int64_t page = c.page_ids[t >> c.log2p];
      const int64_t off = kv_bytes<KV>(page * c.page_stride + int64_t(t & c.pmask) * c.token_stride +
                                       c.head_off + 8 * c.j);
      if constexpr (wide16<KV>())
        ld.v[e] = *reinterpret_cast<const u32x4_t*>(c.vbase + off);
      else if constexpr (nib4<KV>())
        ld.v[e] = *reinterpret_cast<const uint32_t*>(c.vbase + off);
      else
        ld.v[e] = *reinterpret_cast<const uint2*>(c.vbase + off);
    }
  }
  if constexpr (KV == kE4M3T) {
    // Row-wise scales [pages, Hkv, page_size] of this lane's four tokens (of
    // its KV head): with sub-tiles in one page they are four consecutive
    // floats (one 16-byte load each for K and V); otherwise one lookup per
    // token, clamped like the rows themselves.
    const int64_t hrow = c.kvh + c.head_lane;
    if constexpr (PAGE16 && FULL) {
      const int64_t idx =
          ((tp.page * c.num_kv_heads + hrow) << c.log2p) + (t0 & c.pmask) + row_token<HP>(c.q4, 0);
      const float4 k4 = *reinterpret_cast<const float4*>(c.k_scale + idx);
      const float4 v4 = *reinterpret_cast<const float4*>(c.v_scale + idx);
      ld.ks[0] = k4.x, ld.ks[1] = k4.y, ld.ks[2] = k4.z, ld.ks[3] = k4.w;
      ld.vs[0] = v4.x, ld.vs[1] = v4.y, ld.vs[2] = v4.z, ld.vs[3] = v4.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = min(t0 + row_token<HP>(c.q4, e), last);
        const int64_t page = PAGE16 ? tp.page : int64_t(c.page_ids[t >> c.log2p]);
        const int64_t idx = ((page * c.num_kv_heads + hrow) << c.log2p) + (t & c.pmask);
        ld.ks[e] = c.k_scale[idx];
        ld.vs[e] = c.v_scale[idx];
      }
    }
  }
}

// A wavefront tile: nsub<KV>() consecutive sub-tiles, loaded together.
template <int KV>
struct Tile {
  Loads<KV> sub[nsub<KV>()];
};
template <int KV>
struct TileP {
  TilePages sub[nsub<KV>()];
};

template <int KV, bool PAGE16, bool FULL, int HP>
__device__ inline void issue_tile(Tile<KV>& T, const Ctx& c, int t0, const TileP<KV>& tp) {
  constexpr int ST = sub_tokens<HP>();
#pragma unroll
  for (int s = 0; s < nsub<KV>(); ++s) {
    if (FULL || t0 + ST * (s + 1) <= c.kv_len)
      issue_sub<KV, PAGE16, true, HP>(T.sub[s], c, t0 + ST * s, tp.sub[s]);
    else
      issue_sub<KV, PAGE16, false, HP>(T.sub[s], c, t0 + ST * s, tp.sub[s]);
  }
}

// Per-token scale of an e4m3 page (general page sizes); a token past the
// end reads the last token's scale (its weight is 0).
__device__ inline float token_scale(const float* sc, const Ctx& c, const KernelArgs& a, int kvh,
                                    int t) {
  const int tt = min(t, c.kv_len - 1);
  return sc[int64_t(c.page_ids[tt >> c.log2p]) * c.num_kv_heads + kvh];
}

// S = K . q^T of one loaded sub-tile: lane l gets tokens 4*q4 + r of head j.
// The accumulation starts from `init` (int4: minus what the +8 of the widened
// K codes adds to every score of the column, so no per-score correction is
// needed afterwards).
template <int KV>
__device__ inline f32x4_t qk(const Loads<KV>& ld, const u32x4_t (&qb)[q_ops<KV>()],
                             float init = 0.f) {
  f32x4_t s = {init, init, init, init};
  if constexpr (wide16<KV>()) {
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) s = mfma<KV>(ld.k[dc], qb[dc], s);
  } else if constexpr (nib4<KV>()) {
    // two independent accumulation chains (hi and lo parts of q * k_scale)
    f32x4_t s2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) {
      const u32x4_t kb =
          KV == kI4 ? i4x8_to_bf16x8(ld.k[0][dc]) : e2m1x8_to_bf16x8(ld.k[0][dc]);
      s = mfma<KV>(kb, qb[dc], s);
      s2 = mfma<KV>(kb, qb[4 + dc], s2);
    }
    s += s2;
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const u32x4_t w = ld.k[h];
      u32x4_t lo, hi;  // dims 0..7 and 8..15 of the 16 loaded
      lo[0] = e4m3x2_to_bf16x2(w[0], false);
      lo[1] = e4m3x2_to_bf16x2(w[0], true);
      lo[2] = e4m3x2_to_bf16x2(w[1], false);
      lo[3] = e4m3x2_to_bf16x2(w[1], true);
      hi[0] = e4m3x2_to_bf16x2(w[2], false);
      hi[1] = e4m3x2_to_bf16x2(w[2], true);
      hi[2] = e4m3x2_to_bf16x2(w[3], false);
      hi[3] = e4m3x2_to_bf16x2(w[3], true);
      s = mfma<KV>(lo, qb[2 * h], s);
      s = mfma<KV>(hi, qb[2 * h + 1], s);
    }
  }
  return s;
}

// Scores in log2 units (sm_scale, and e4m3 K scales, applied), -inf past the
// row's causal limit; `grow` is set when one exceeds the reference max by more
// than the slack.
template <int KV, bool PAGE16, bool FULL, int HP>
__device__ inline void scale_mask(const f32x4_t& s, const Loads<KV>& ld, const Ctx& c,
                                  const KernelArgs& a, int kvh, int t0, const TilePages& tp,
                                  int lim, bool cross, float m_run, float (&sc)[4], bool& grow) {
  float ks = a.sm_scale_log2;
  if constexpr (KV == kE4M3 && PAGE16) ks *= tp.ks;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = t0 + row_token<HP>(c.q4, r);
    float kr = ks;
    if constexpr (KV == kE4M3 && !PAGE16) kr = ks * token_scale(a.k_scale, c, a, kvh, t);
    if constexpr (KV == kE4M3T) kr = ks * ld.ks[r];
    const bool ok = (FULL || t < lim) && (HP == 1 || !cross);
    const float v = ok ? s[r] * kr : -INFINITY;
    sc[r] = v;
    grow |= v > m_run + kSlack;
  }
}

// Lazy reference max: p = 2^(s - m) may reach 2^kSlack; only when a score
// exceeds that does the wavefront move m (to the exact running max of each
// head) and rescale d and O by 2^(m_old - m_new). The first tile always moves
// it (m starts at -inf). Results do not depend on m beyond rounding.
template <bool FULL, int N>
__device__ inline void move_max(const float (&sc)[N][4], const Ctx& c, bool grow,
                                f32x4_t (&acc)[8], float& m_run, float& d_run) {
  if (__any(grow)) {
    float mt = -INFINITY;
#pragma unroll
    for (int n = 0; n < N; ++n)
      mt = fmaxf(mt, fmaxf(fmaxf(sc[n][0], sc[n][1]), fmaxf(sc[n][2], sc[n][3])));
    mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    // 0 while m_run = -inf; a masked tile can leave a row without any token
    // yet (m_new = -inf), whose d and O are still 0: no rescale.
    float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    if constexpr (!FULL) alpha = m_new == -INFINITY ? 1.f : alpha;
    m_run = m_new;
    d_run *= alpha;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float ar = __shfl(alpha, 4 * c.q4 + r, 64);
#pragma unroll
      for (int nc = 0; nc < 8; ++nc) acc[nc][r] *= ar;
    }
  }
}

// P of one sub-tile as hi + lo 16-bit pairs (k-slot e of quarter q4 is token
// 4*q4 + e), its sum added to d, and e4m3 V scales folded in.
template <int KV, bool PAGE16, bool FULL, int HP>
__device__ inline void probs(const float (&sc)[4], const Loads<KV>& ld, const Ctx& c,
                             const KernelArgs& a, int kvh, int t0, const TilePages& tp,
                             float m_run, float& d_run, uint2& p_hi, uint2& p_lo) {
  float p[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    p[e] = __builtin_amdgcn_exp2f(sc[e] - m_run);
    // masked scores give 0, also when m_run = -inf (head pairs mask the
    // other head's lanes in full tiles too, while m_run is already finite)
    if constexpr (!FULL) p[e] = sc[e] == -INFINITY ? 0.f : p[e];
    d_run += p[e];
  }
  if constexpr (KV == kE4M3) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float vs;
      if constexpr (PAGE16)
        vs = tp.vs;
      else
        vs = token_scale(a.v_scale, c, a, kvh, t0 + 4 * c.q4 + e);
      p[e] *= vs;
    }
  }
  if constexpr (KV == kE4M3T) {
#pragma unroll
    for (int e = 0; e < 4; ++e) p[e] *= ld.vs[e];
  }
  split16<KV>(p[0], p[1], p_hi.x, p_lo.x);
  split16<KV>(p[2], p[3], p_hi.y, p_lo.y);
}

// V as the B operand of P.V for output columns nc: four 16-bit values,
// V[token 4*q4 + e][dim 8*j + nc] for e = 0..3 (nc is a constant after
// unrolling).
template <int KV>
__device__ inline uint2 v_operand(const Loads<KV>& ld, int nc) {
  static_assert(KV != kI4, "int4 V operands come from i4_v_words");
  uint2 vb;
  if constexpr (wide16<KV>()) {
    const int w = nc >> 1;
    const bool hi = nc & 1;
    vb.x = pack_halves(ld.v[0][w], ld.v[1][w], hi);
    vb.y = pack_halves(ld.v[2][w], ld.v[3][w], hi);
  } else if constexpr (nib4<KV>()) {
    // byte nc/2 of each token's word holds dims 8*j + nc (nibble nc&1)
    const bool hi = nc & 1;
    uint32_t x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      switch (nc >> 1) {
        case 0: x[e] = e2m1x2_to_bf16x2<0>(ld.v[e]); break;
        case 1: x[e] = e2m1x2_to_bf16x2<1>(ld.v[e]); break;
        case 2: x[e] = e2m1x2_to_bf16x2<2>(ld.v[e]); break;
        default: x[e] = e2m1x2_to_bf16x2<3>(ld.v[e]); break;
      }
    }
    vb.x = pack_halves(x[0], x[1], hi);
    vb.y = pack_halves(x[2], x[3], hi);
  } else {
    const int w = nc >> 2;           // word of the 8 loaded bytes
    const bool hiw = (nc >> 1) & 1;  // which byte pair in the word
    const bool hib = nc & 1;         // which byte of the pair
    uint32_t x[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = e4m3x2_to_bf16x2(w ? ld.v[e].y : ld.v[e].x, hiw);
    vb.x = pack_halves(x[0], x[1], hib);
    vb.y = pack_halves(x[2], x[3], hib);
  }
  return vb;
}

#ifndef PKD_FP4_VT
#define PKD_FP4_VT 1
#endif
// e2m1 V of one sub-tile regrouped for P.V: the four token words of a lane
// (dims 8*j..+8 of tokens 4*q4 + e) interleaved nibble by nibble in pairs of
// tokens, so that byte b of w[2*h + o] holds dim 8*j + 2*b + o of tokens
// 2*h (low nibble) and 2*h + 1 (high nibble): one conversion then yields
// the two bf16 values of a B-operand word.
struct VPairs {
  uint32_t w[4];
};
__device__ inline VPairs fp4_v_pairs(const uint32_t (&v)[4]) {
  constexpr uint32_t kLo = 0x0F0F0F0Fu;
  VPairs r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t a = v[2 * h], b = v[2 * h + 1];
    r.w[2 * h] = (a & kLo) | ((b << 4) & ~kLo);      // even dims
    r.w[2 * h + 1] = ((a >> 4) & kLo) | (b & ~kLo);  // odd dims
  }
  return r;
}
__device__ inline uint2 fp4_v_operand(const VPairs& vp, int nc) {
  const int o = nc & 1;
  uint2 vb;
  switch (nc >> 1) {
    case 0: vb.x = e2m1x2_to_bf16x2<0>(vp.w[o]), vb.y = e2m1x2_to_bf16x2<0>(vp.w[2 + o]); break;
    case 1: vb.x = e2m1x2_to_bf16x2<1>(vp.w[o]), vb.y = e2m1x2_to_bf16x2<1>(vp.w[2 + o]); break;
    case 2: vb.x = e2m1x2_to_bf16x2<2>(vp.w[o]), vb.y = e2m1x2_to_bf16x2<2>(vp.w[2 + o]); break;
    default: vb.x = e2m1x2_to_bf16x2<3>(vp.w[o]), vb.y = e2m1x2_to_bf16x2<3>(vp.w[2 + o]); break;
  }
  return vb;
}

// int4 V of one sub-tile for P.V: the four token words of a lane (dims
// 8*j..+8 of tokens 4*q4 + e) as unsigned k = code + 8 in the low nibble of
// bytes, the bytes of tokens 2h and 2h + 1 side by side, so that one fp8
// conversion (see i4x8_to_bf16x8) yields a B-operand word: w[h][x] holds
// dims (2i, 2i') of tokens (2h, 2h + 1) from the low nibbles (x = 0: i = 0,
// i' = 1; x = 1: i = 2, i' = 3) and dims (2i + 1, 2i' + 1) from the high
// nibbles (x = 2, 3).
struct I4Words {
  uint32_t w[2][4];
};
__device__ inline I4Words i4_v_words(const uint32_t (&v)[4]) {
  I4Words r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t a = v[2 * h] ^ 0x88888888u, b = v[2 * h + 1] ^ 0x88888888u;
    const uint32_t alo = a & 0x0F0F0F0Fu, ahi = (a >> 4) & 0x0F0F0F0Fu;
    const uint32_t blo = b & 0x0F0F0F0Fu, bhi = (b >> 4) & 0x0F0F0F0Fu;
    // bytes (a.i, b.i, a.i', b.i'): selector bytes 0-3 pick the second
    // operand's bytes, 4-7 the first's
    r.w[h][0] = __builtin_amdgcn_perm(blo, alo, 0x05010400u);
    r.w[h][1] = __builtin_amdgcn_perm(blo, alo, 0x07030602u);
    r.w[h][2] = __builtin_amdgcn_perm(bhi, ahi, 0x05010400u);
    r.w[h][3] = __builtin_amdgcn_perm(bhi, ahi, 0x07030602u);
  }
  return r;
}
// B operand of output columns nc (dim 8*j + nc): (k * 2^-9) of tokens 0, 1
// and 2, 3.
__device__ inline uint2 i4_v_operand(const I4Words& iw, int nc) {
  const int x = (nc & 1 ? 2 : 0) + ((nc >> 2) & 1);
  const bool second = (nc >> 1) & 1;  // dim 2i' of the word's pair of dims
  return uint2{e4m3x2_to_bf16x2(iw.w[0][x], second), e4m3x2_to_bf16x2(iw.w[1][x], second)};
}

// Per column group (16 S columns each; two groups when a work item carries
// 17-32 query rows): the q operands, the running softmax state and O of the
// lane's column, and the tokens that column's row sees. Both groups consume
// the same K and V loads and the same V operands.
template <int KV, int NG>
struct Groups {
  u32x4_t qb[NG][q_ops<KV>()];
  f32x4_t acc[NG][8];
  float m_run[NG];  // reference max (log2 units), uniform over quarters
  float d_run[NG];  // sum of p over this lane's tokens
  float s0[NG];     // start of the score accumulation (int4: minus what the +8 of the K codes adds)
  int lim[NG];      // tokens of the item seen by this lane's row (column j of S)
  bool cross[NG];   // head pairs: the lane's S rows are not its column's head (masked)
};

// QK, online softmax and PV for one loaded sub-tile (FULL: all 16 tokens
// valid); P.V on the k = 16 MFMA.
template <int KV, bool PAGE16, bool FULL, int HP, int NG>
__device__ inline void process_sub(const Loads<KV>& ld, const Ctx& c, const KernelArgs& a, int kvh,
                                    int t0, const TilePages& tp, Groups<KV, NG>& gs) {
  uint2 p_hi[NG], p_lo[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const f32x4_t s = qk<KV>(ld, gs.qb[g], KV == kI4 ? gs.s0[g] : 0.f);
    float sc[1][4];
    bool grow = false;
    scale_mask<KV, PAGE16, FULL, HP>(s, ld, c, a, kvh, t0, tp, gs.lim[g], gs.cross[g],
                                     gs.m_run[g], sc[0], grow);
    move_max<FULL, 1>(sc, c, grow, gs.acc[g], gs.m_run[g], gs.d_run[g]);
    probs<KV, PAGE16, FULL, HP>(sc[0], ld, c, a, kvh, t0, tp, gs.m_run[g], gs.d_run[g], p_hi[g],
                                p_lo[g]);
  }
  // O += P . V, column j of MFMA nc is dim 8*j + nc
#pragma unroll
  for (int nc = 0; nc < 8; ++nc) {
    const uint2 vb = v_operand<KV>(ld, nc);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      gs.acc[g][nc] = mfma16<KV>(p_hi[g], vb, gs.acc[g][nc]);
      gs.acc[g][nc] = mfma16<KV>(p_lo[g], vb, gs.acc[g][nc]);
    }
  }
}

// Two consecutive sub-tiles A and B at once: their 32 tokens share one
// reference-max update and feed P.V on the k = 32 MFMA, whose k-slots
// 8*q4 + e are token 4*q4 + e of A (e < 4) and 4*q4 + e - 4 of B, so the A
// and B operands are the two sub-tiles' k = 16 operands side by side (half
// the P.V instructions of two k = 16 passes).
template <int KV, bool PAGE16, bool FULL, int HP, int NG>
__device__ inline void process_pair(const Loads<KV>& la, const Loads<KV>& lb, const Ctx& c,
                                    const KernelArgs& a, int kvh, int t0, const TilePages& ta,
                                    const TilePages& tb, Groups<KV, NG>& gs) {
  constexpr int ST = sub_tokens<HP>();
  u32x4_t p_hi[NG], p_lo[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const f32x4_t sa = qk<KV>(la, gs.qb[g], KV == kI4 ? gs.s0[g] : 0.f);
    const f32x4_t sb = qk<KV>(lb, gs.qb[g], KV == kI4 ? gs.s0[g] : 0.f);
    float sc[2][4];
    bool grow = false;
    scale_mask<KV, PAGE16, FULL, HP>(sa, la, c, a, kvh, t0, ta, gs.lim[g], gs.cross[g],
                                     gs.m_run[g], sc[0], grow);
    scale_mask<KV, PAGE16, FULL, HP>(sb, lb, c, a, kvh, t0 + ST, tb, gs.lim[g], gs.cross[g],
                                     gs.m_run[g], sc[1], grow);
    move_max<FULL, 2>(sc, c, grow, gs.acc[g], gs.m_run[g], gs.d_run[g]);
    uint2 pa_hi, pa_lo, pb_hi, pb_lo;
    probs<KV, PAGE16, FULL, HP>(sc[0], la, c, a, kvh, t0, ta, gs.m_run[g], gs.d_run[g], pa_hi,
                                pa_lo);
    probs<KV, PAGE16, FULL, HP>(sc[1], lb, c, a, kvh, t0 + ST, tb, gs.m_run[g], gs.d_run[g],
                                pb_hi, pb_lo);
    p_hi[g] = u32x4_t{pa_hi.x, pa_hi.y, pb_hi.x, pb_hi.y};
    p_lo[g] = u32x4_t{pa_lo.x, pa_lo.y, pb_lo.x, pb_lo.y};
  }
  VPairs vpa, vpb;
  I4Words ia, ib;
  if constexpr (KV == kE2M1 && PKD_FP4_VT) {
    vpa = fp4_v_pairs(la.v);
    vpb = fp4_v_pairs(lb.v);
  }
  if constexpr (KV == kI4) {
    ia = i4_v_words(la.v);
    ib = i4_v_words(lb.v);
  }
#pragma unroll
  for (int nc = 0; nc < 8; ++nc) {
    uint2 va, vb;
    if constexpr (KV == kI4) {
      va = i4_v_operand(ia, nc);
      vb = i4_v_operand(ib, nc);
    } else if constexpr (KV == kE2M1 && PKD_FP4_VT) {
      va = fp4_v_operand(vpa, nc);
      vb = fp4_v_operand(vpb, nc);
    } else {
      va = v_operand<KV>(la, nc);
      vb = v_operand<KV>(lb, nc);
    }
    const u32x4_t v = {va.x, va.y, vb.x, vb.y};
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      gs.acc[g][nc] = mfma<KV>(p_hi[g], v, gs.acc[g][nc]);
      gs.acc[g][nc] = mfma<KV>(p_lo[g], v, gs.acc[g][nc]);
    }
  }
}

#ifndef PKD_PAIR_PV
#define PKD_PAIR_PV 1
#endif

template <int KV, bool PAGE16, bool FULL, int HP, int NG>
__device__ inline void process_tile(const Tile<KV>& T, const Ctx& c, const KernelArgs& a, int kvh,
                                    int t0, const TileP<KV>& tp, Groups<KV, NG>& gs) {
  constexpr int NS = nsub<KV>();
  constexpr int ST = sub_tokens<HP>();
  if constexpr (PKD_PAIR_PV && NS % 2 == 0) {
#pragma unroll
    for (int s = 0; s < NS; s += 2)
      process_pair<KV, PAGE16, FULL, HP, NG>(T.sub[s], T.sub[s + 1], c, a, kvh, t0 + ST * s,
                                             tp.sub[s], tp.sub[s + 1], gs);
  } else {
#pragma unroll
    for (int s = 0; s < NS; ++s)
      process_sub<KV, PAGE16, FULL, HP, NG>(T.sub[s], c, a, kvh, t0 + ST * s, tp.sub[s], gs);
  }
}

// Page ids (and e4m3 scales) of a block of consecutive tiles of one
// wavefront, one sub-tile per lane (64 sub-tiles per block); read back with
// readlane. A sub-tile past the item's end takes the last sub-tile's page.
template <int KV>
constexpr int pid_block_tiles() { return 64 / nsub<KV>(); }

struct PidBlock {
  int32_t pid = 0;
  float ks[2] = {1.f, 1.f};  // e4m3: the page's scales of the workgroup's KV heads
  float vs[2] = {1.f, 1.f};
};

template <int KV, int HP>
__device__ inline void load_pid_block(const Ctx& c, int wave, int first_tile, int lane,
                                      PidBlock& b) {
  constexpr int ST = sub_tokens<HP>();
  const int tile = first_tile + lane / nsub<KV>();
  const int t = (wave + kWaves * tile) * tile_tokens<KV, HP>() + ST * (lane % nsub<KV>());
  const int tt = min(t, (c.kv_len - 1) & ~(ST - 1));
  b.pid = c.page_ids[tt >> c.log2p];
  if constexpr (KV == kE4M3) {
    const int64_t idx = int64_t(b.pid) * c.num_kv_heads + c.kvh;
#pragma unroll
    for (int h = 0; h < HP; ++h) {
      b.ks[h] = c.k_scale[idx + h];
      b.vs[h] = c.v_scale[idx + h];
    }
  }
}

// Register budget: up to 168 VGPRs (3 wavefronts per SIMD) by default, as
// one workgroup of four wavefronts per CU (the default residency) leaves
// room for; row-wise e4m3 scales ride along with the loads and get up to 256
// (2 per SIMD), as do e2m1 (four sub-tiles and the q hi/lo pair in flight),
// head pairs (two scales per page for e4m3), two column groups and e4m3 or
// int4 with pages under 16 tokens (per-lane page lookups). int4 (the
// most VALU work per byte) gets 168 so that three workgroups fit a CU (its
// 4 KiB tiles need 159-165 with the persistent unit loop).
template <int KV, bool PAGE16, int HP, int G>
constexpr int waves_per_simd() {
  if constexpr (KV == kI4) return G <= 16 && PAGE16 ? 3 : 2;
  return KV == kE4M3T || nib4<KV>() || HP > 1 || G > 16 || (fp8<KV>() && !PAGE16) ? 2 : 3;
}

// One work unit: work item `item` (a run of one request's pages for a block
// of its query tokens) for KV head (pair) kvh, from its query rows to its
// output rows or partial states. Called by every thread of the workgroup;
// `st` is the workgroup's shared state image. Persistent launches: thread 0
// takes the workgroup's next unit when this one's tiles are done (so units are
// handed out in the order workgroups become free) and returns it.
template <int KV, int G, bool PAGE16, int HP>
__device__ inline int decode_unit(const KernelArgs& a, WaveStates<G, kD>& st, int item, int kvh) {
  constexpr int NG = G > 16 ? 2 : 1;  // column groups of 16
  const DeviceItem it = a.items[item];
  // The lane index is opaque (opaque_tid) so that nothing derived from it
  // (lane offsets, masks) is computed once for all the units of a persistent
  // workgroup and held in registers across them.
  const int tid = opaque_tid();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  Ctx c;
  c.kbase = static_cast<const char*>(a.k);
  c.vbase = static_cast<const char*>(a.v);
  c.page_ids = a.indices + it.page_begin;
  c.k_scale = a.k_scale;
  c.v_scale = a.v_scale;
  c.num_kv_heads = a.num_kv_heads * HP;
  c.kvh = kvh * HP;  // first (or only) KV head of this workgroup
  c.page_stride = a.page_stride;
  c.token_stride = a.token_stride;
  c.head_stride = a.head_stride;
  c.head_off = int64_t(c.kvh) * a.head_stride;
  c.kbase_h = c.kbase + kv_bytes<KV>(c.head_off);
  c.vbase_h = c.vbase + kv_bytes<KV>(c.head_off);
  c.page_bytes = uint32_t(kv_bytes<KV>(a.page_stride));
  c.token_bytes = uint32_t(kv_bytes<KV>(a.token_stride));
  c.log2p = a.page_size_log2;
  c.pmask = (1 << a.page_size_log2) - 1;
  c.kv_len = it.kv_len;
  c.q4 = lane >> 4;
  c.j = lane & 15;
  Groups<KV, NG> gs;
  // Column j of group g is row rho = 16*g + j of the item: query token qi of
  // the item's block, query head kvh*group + hh. Head pairs: the column's
  // head is hh / (query heads per KV head); the lane's rows' head is q4 / 2.
  constexpr int HPL = HP == 1 ? 0 : 1;
  constexpr int STL = sub_tokens_log2<HP>();
  c.head_lane = row_head<HP>(c.q4);
  if constexpr (HP > 1) {
    c.koff = uint32_t(kv_bytes<KV>(int64_t(c.j & ((1 << STL) - 1)) * a.token_stride +
                                   (c.j >> STL) * a.head_stride + qk_dim<KV>(0, c.q4, 0)));
    c.voff = uint32_t(kv_bytes<KV>(int64_t(row_token<HP>(c.q4, 0)) * a.token_stride +
                                   c.head_lane * a.head_stride + 8 * c.j));
  } else {
    c.koff = uint32_t(kv_bytes<KV>(int64_t(c.j) * a.token_stride + qk_dim<KV>(0, c.q4, 0)));
    c.voff = uint32_t(kv_bytes<KV>(int64_t(4 * c.q4) * a.token_stride + 8 * c.j));
  }
  c.vrow_bytes = kv_bytes<KV>(a.token_stride);

  // q^T as the B operand of S = K.q^T: column j of group g = row 16*g + j
  // (zero beyond the block): eight 16-bit q values per k step (bf16, or fp16
  // for fp16 KV).
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int rho = 16 * g + c.j;
    const int qi = rho >> a.group_log2;
    const int hh = rho & ((1 << a.group_log2) - 1);
    const bool row_ok = rho < G && qi < it.q_len;
    gs.lim[g] = row_ok ? min(it.kv_len, it.visible + qi) : it.kv_len;
    const int col_head = HP == 1 ? 0 : hh >> (a.group_log2 - HPL);
    gs.cross[g] = HP > 1 && c.head_lane != col_head;
    u32x4_t (&qb)[q_ops<KV>()] = gs.qb[g];
    float qsum = 0.f;  // int4: sum of this lane's q' (hi + lo as fed)
    const uint16_t* qp =
        static_cast<const uint16_t*>(a.q) +
        (int64_t(it.q_row + qi) * a.num_qo_heads + (int64_t(kvh) << a.group_log2) + hh) * kD;
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) {
      u32x4_t w = {0u, 0u, 0u, 0u};
      if (row_ok) w = *reinterpret_cast<const u32x4_t*>(qp + qk_dim<KV>(dc, c.q4, 0));
      if constexpr (nib4<KV>()) {
        // q * k_scale over this step's eight dims, as hi + lo bf16
        const float* ksp = a.k_scale + int64_t(c.kvh + col_head) * kD + qk_dim<KV>(dc, c.q4, 0);
        const float4 s0 = *reinterpret_cast<const float4*>(ksp);
        const float4 s1 = *reinterpret_cast<const float4*>(ksp + 4);
        const float ksv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        u32x4_t hi, lo;
        if constexpr (KV == kI4) {
          // q' = q * k_scale * 2^9 (the widened K codes carry 2^-9), in the
          // dim order of i4x8_to_bf16x8: words (0, 2), (4, 6), (1, 3), (5, 7)
          float qf[8];
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            qf[2 * x] = __builtin_bit_cast(float, w[x] << 16) * ksv[2 * x] * 512.f;
            qf[2 * x + 1] = __builtin_bit_cast(float, w[x] & 0xffff0000u) * ksv[2 * x + 1] * 512.f;
          }
          constexpr int kOrd[8] = {0, 2, 4, 6, 1, 3, 5, 7};
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            uint32_t h, l;
            split16<KV>(qf[kOrd[2 * x]], qf[kOrd[2 * x + 1]], h, l);
            hi[x] = h;
            lo[x] = l;
            qsum += (__builtin_bit_cast(float, h << 16) + __builtin_bit_cast(float, l << 16)) +
                    (__builtin_bit_cast(float, h & 0xffff0000u) +
                     __builtin_bit_cast(float, l & 0xffff0000u));
          }
        } else {
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            const float q0 = __builtin_bit_cast(float, w[x] << 16) * ksv[2 * x];
            const float q1 = __builtin_bit_cast(float, w[x] & 0xffff0000u) * ksv[2 * x + 1];
            uint32_t h, l;
            split16<KV>(q0, q1, h, l);
            hi[x] = h;
            lo[x] = l;
          }
        }
        qb[dc] = hi;
        qb[4 + dc] = lo;
      } else {
        qb[dc] = w;
      }
    }
    // int4: the K operand is (code + 8) * 2^-9, so each score carries
    // 8 * 2^-9 * (sum of q' over all 128 dims); the four quarters of a
    // column hold 32 dims each
    qsum += __shfl_xor(qsum, 16, 64);
    qsum += __shfl_xor(qsum, 32, 64);
    gs.s0[g] = KV == kI4 ? -qsum * (1.f / 64.f) : 0.f;
  }

#pragma unroll
  for (int g = 0; g < NG; ++g) {
#pragma unroll
    for (int nc = 0; nc < 8; ++nc) gs.acc[g][nc] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    gs.m_run[g] = -INFINITY;
    gs.d_run[g] = 0.f;
  }

  // Tiles of this wavefront: tokens [(wave + 4i) * TT, +TT) for i < n, with
  // TT = tile_tokens<KV, HP>().
  constexpr int TT = tile_tokens<KV, HP>();
  constexpr int NS = nsub<KV>();
  constexpr int kBlk = pid_block_tiles<KV>();
  const int first = wave * TT;
  const int n = first < c.kv_len ? (c.kv_len - first + kWaves * TT - 1) / (kWaves * TT) : 0;
  if (n > 0) {
    PidBlock blk_cur, blk_next;
    if constexpr (PAGE16) {
      load_pid_block<KV, HP>(c, wave, 0, lane, blk_cur);
      if (n > kBlk) load_pid_block<KV, HP>(c, wave, kBlk, lane, blk_next);
    }
    auto lane_float = [](float x, int slot) {
      return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), slot));
    };
    // Pages of tile i (tiles are issued in order, so the id block only moves forward).
    auto pages_of = [&](int i) {
      TileP<KV> tp;
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2) {
        tp.sub[s2].page = 0;
        tp.sub[s2].ks = tp.sub[s2].vs = 1.f;
      }
      if constexpr (PAGE16) {
        if (i > 0 && (i % kBlk) == 0) {
          blk_cur = blk_next;
          if (i + kBlk < n) load_pid_block<KV, HP>(c, wave, i + kBlk, lane, blk_next);
        }
#pragma unroll
        for (int s2 = 0; s2 < NS; ++s2) {
          const int slot = (i % kBlk) * NS + s2;
          tp.sub[s2].page = __builtin_amdgcn_readlane(blk_cur.pid, slot);
          if constexpr (KV == kE4M3) {
            // the workgroup's heads' scales (uniform), then this lane's head's
#pragma unroll
            for (int h = 0; h < HP; ++h) {
              const float ksh = lane_float(blk_cur.ks[h], slot);
              const float vsh = lane_float(blk_cur.vs[h], slot);
              if (h == 0 || c.head_lane == h) {
                tp.sub[s2].ks = ksh;
                tp.sub[s2].vs = vsh;
              }
            }
          }
        }
      }
      return tp;
    };
    auto tok = [&](int i) { return first + i * kWaves * TT; };

    // Two tile buffers: tile i + 1 is in flight while tile i is computed. Inside
    // the loop the next tile is always issued (full-tile code only) before the
    // current one is computed, so the wait before each tile's math covers
    // exactly that tile's loads. Only a wavefront's last tile can be partial;
    // it is issued and computed after the loop.
    Tile<KV> cur, nxt;
    TileP<KV> pc = pages_of(0), pn;
    const int h0 = c.kvh;
    if (n == 1) {
      issue_tile<KV, PAGE16, false, HP>(cur, c, tok(0), pc);
      process_tile<KV, PAGE16, false, HP, NG>(cur, c, a, h0, tok(0), pc, gs);
    } else {
      issue_tile<KV, PAGE16, true, HP>(cur, c, tok(0), pc);
      for (int i = 0; i + 2 < n; ++i) {
        pn = pages_of(i + 1);
        issue_tile<KV, PAGE16, true, HP>(nxt, c, tok(i + 1), pn);
        process_tile<KV, PAGE16, true, HP, NG>(cur, c, a, h0, tok(i), pc, gs);
        cur = nxt;
        pc = pn;
      }
      pn = pages_of(n - 1);
      issue_tile<KV, PAGE16, false, HP>(nxt, c, tok(n - 1), pn);
      process_tile<KV, PAGE16, true, HP, NG>(cur, c, a, h0, tok(n - 2), pc, gs);
      process_tile<KV, PAGE16, false, HP, NG>(nxt, c, a, h0, tok(n - 1), pn, gs);
    }
  }

  // ---- per-wavefront state -> shared memory
  const int q4 = c.q4, j = c.j;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    f32x4_t (&acc)[8] = gs.acc[g];
    float d_run = gs.d_run[g];
    d_run += __shfl_xor(d_run, 16, 64);
    d_run += __shfl_xor(d_run, 32, 64);
    if constexpr (nib4<KV>()) {
      // V channel scales: column j of MFMA nc is dim 8*j + nc, of the KV head
      // of O row 4*q4 + r (row / query heads per KV head, within the pair)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int hrow = (16 * g + 4 * q4 + r) & ((1 << a.group_log2) - 1);
        const int hsel = HP == 1 ? 0 : hrow >> (a.group_log2 - HPL);
        const float* vsp = a.v_scale + int64_t(c.kvh + hsel) * kD + 8 * j;
        const float4 s0 = *reinterpret_cast<const float4*>(vsp);
        const float4 s1 = *reinterpret_cast<const float4*>(vsp + 4);
        const float vsv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
        if constexpr (KV == kI4) {
          // O holds sum P * (code + 8) * 2^-9 for row 4*q4 + r, whose d
          // (the sum of P, in column lane 4*q4 + r) removes the + 8. P.V
          // takes P as hi + lo bf16 parts, within 2^-17 of P, so what is
          // left of the + 8 after normalising is below 8 * 2^-17 of one
          // code step (v_scale)
          const float dr = __shfl(d_run, 4 * q4 + r, 64) * (1.f / 64.f);
#pragma unroll
          for (int nc = 0; nc < 8; ++nc) acc[nc][r] = (acc[nc][r] - dr) * (vsv[nc] * 512.f);
        } else {
#pragma unroll
          for (int nc = 0; nc < 8; ++nc) acc[nc][r] *= vsv[nc];
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = 16 * g + 4 * q4 + r;
      if (h < G) {
#pragma unroll
        for (int nc = 0; nc < 8; ++nc) st.o[wave][h][8 * j + nc] = acc[nc][r];
      }
    }
    if (q4 == 0 && 16 * g + j < G) {
      st.m[wave][16 * g + j] = gs.m_run[g];
      st.d[wave][16 * g + j] = d_run;
    }
  }
  __syncthreads();
  int next = 0;
  if (a.persistent && tid == 0) next = int(gridDim.x) + atomicAdd(a.work, 1);
  finish_workgroup<G, kD>(st, a, it, kvh);
  return next;
}

// G: S columns (query rows) per workgroup. HP = 2: the workgroup's "KV head"
// kvh of the launch is a pair of KV heads 2*kvh, 2*kvh + 1 with G / 2 query
// heads each (the launch passes num_kv_heads / 2 and group_log2 + 1, so the
// epilogue and the merge address query heads as usual).
//
// Work units are (item, KV head (pair)) in plan order. A plain launch runs
// one unit per workgroup (decode_block). A persistent launch runs the
// device's resident workgroups, each taking units from a counter until none
// is left: the longest units still start first, every compute unit takes the
// next unit as soon as it is free (a plain launch hands workgroup ids to the
// eight XCDs in turn, so a free compute unit can idle until an id for its XCD
// comes up), and no workgroup waits for another (the counters are only ever
// incremented), so every workgroup exits.
template <int KV, int G, bool PAGE16, int HP>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(waves_per_simd<KV, PAGE16, HP, G>()))) void decode_mfma_kernel(KernelArgs a) {
  static_assert(G >= 1 && G <= 32, "at most 32 query rows per KV head");
  static_assert(HP == 1 || (G >= HP && PAGE16), "head pairs: pages >= 16");
  __shared__ WaveStates<G, kD> st;
  __shared__ int s_next;

  if (!a.persistent) {
    int item, kvh;
    decode_block(a.num_kv_heads, a.xcd_group, &item, &kvh);
    if (item >= launch_items(a)) return;  // grid padding; no barrier passed yet
    decode_unit<KV, G, PAGE16, HP>(a, st, item, kvh);
    return;
  }
  const int units = launch_items(a) * a.num_kv_heads;
  for (int u = blockIdx.x; u < units;) {
    const int item = u / a.num_kv_heads;
    const int next = decode_unit<KV, G, PAGE16, HP>(a, st, item, u - item * a.num_kv_heads);
    if (threadIdx.x == 0) s_next = next;
    __syncthreads();  // also: the next unit writes st only after every read of this one
    u = s_next;
    __syncthreads();
  }
  // The last workgroup to finish resets the counters (by then every
  // workgroup has made its last fetch).
  if (threadIdx.x == 0 && atomicAdd(a.work + 1, 1) == int(gridDim.x) - 1) {
    __hip_atomic_store(a.work, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.work + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int KV, bool P16>
DecodeFn pick_group(int g) {
  switch (g) {
    case 1: return decode_mfma_kernel<KV, 1, P16, 1>;
    case 2: return decode_mfma_kernel<KV, 2, P16, 1>;
    case 4: return decode_mfma_kernel<KV, 4, P16, 1>;
    case 8: return decode_mfma_kernel<KV, 8, P16, 1>;
    case 16: return decode_mfma_kernel<KV, 16, P16, 1>;
    case 32:  // two column groups (not 4-bit KV: its q hi/lo pairs would not fit the registers)
      if constexpr (!nib4<KV>()) return decode_mfma_kernel<KV, 32, P16, 1>;
      return nullptr;
    default: return nullptr;
  }
}

// Pairs of KV heads per workgroup: `cols` = 2 x the rows of one head.
template <int KV>
DecodeFn pick_pair(int cols) {
  switch (cols) {
    case 2: return decode_mfma_kernel<KV, 2, true, 2>;
    case 4: return decode_mfma_kernel<KV, 4, true, 2>;
    case 8: return decode_mfma_kernel<KV, 8, true, 2>;
    case 16: return decode_mfma_kernel<KV, 16, true, 2>;
    case 32:  // two column groups (not 4-bit KV, as for one head)
      if constexpr (!nib4<KV>()) return decode_mfma_kernel<KV, 32, true, 2>;
      return nullptr;
    default: return nullptr;
  }
}

}  // namespace

DecodeFn mfma_decode_kernel(int kv_dtype, int head_dim, int rows, int page_size, int hp) {
  if (head_dim != kD) return nullptr;
  const bool p16 = page_size >= 16;

  if (hp == 2) {
    if (!p16) return nullptr;
    switch (kv_dtype) {
      case kBF16: return pick_pair<kBF16>(rows);
      case kE4M3: return pick_pair<kE4M3>(rows);
      case kE4M3T: return pick_pair<kE4M3T>(rows);
      case kF16: return pick_pair<kF16>(rows);
      case kE2M1: return pick_pair<kE2M1>(rows);
      case kI4: return pick_pair<kI4>(rows);
      default: return nullptr;
    }
  }
  if (hp != 1) return nullptr;
  switch (kv_dtype) {
    case kBF16: return p16 ? pick_group<kBF16, true>(rows) : pick_group<kBF16, false>(rows);
    case kE4M3: return p16 ? pick_group<kE4M3, true>(rows) : pick_group<kE4M3, false>(rows);
    case kE4M3T: return p16 ? pick_group<kE4M3T, true>(rows) : pick_group<kE4M3T, false>(rows);
    case kF16: return p16 ? pick_group<kF16, true>(rows) : pick_group<kF16, false>(rows);
    case kE2M1: return p16 ? pick_group<kE2M1, true>(rows) : pick_group<kE2M1, false>(rows);
    case kI4: return p16 ? pick_group<kI4, true>(rows) : pick_group<kI4, false>(rows);
    default: return nullptr;
  }
}

}  // namespace pkd
