// Persistent split-KV decode attention over a paged KV cache.
//
// Method (SGLang x HPC-Ops page, "Scheduling around live KV work", second
// paragraph; vLLM x HPC-Ops page, bullet "Compute and combine"): one
// resident workgroup per bin walks its task descriptors in order; for each
// descriptor (KV head g, request r, tokens [a, e)) it computes attention of
// the KV head's whole query group over those tokens and writes a partial
// output with its log-sum-exp, then moves on to the next descriptor without
// a relaunch.
//
// gfx950 mapping (our design, not the pages'):
//  * A workgroup is W waves (8 for BF16 KV and for FP8 KV with an FP8
//    query, 6 for FP8 KV with a BF16 query).  A descriptor's tokens are cut
//    into 16-token slices (a slice never crosses a 64-token page because
//    descriptors start on page boundaries); slice i goes to wave i % W.  Each
//    wave keeps its own running max, sum and output for the group, so there
//    is no barrier inside a descriptor; the W states are merged through LDS
//    at its end.
//  * Scores use MFMA 16x16x32 bf16 with the 16 slice tokens as rows and the
//    query heads as columns (S^T = K Q^T; G <= 16 heads, unused columns are
//    zero).  P.V uses MFMA 16x16x16 bf16 as O^T = V^T P^T, whose B operand
//    is exactly the score accumulator layout, so probabilities never leave
//    registers.
//  * K rows are loaded straight into the MFMA A layout (each lane 16 B of
//    one token).  V is loaded 4 tokens x 256 contiguous bytes per
//    instruction (lane = 8 dims of one token); the contraction over tokens
//    is order-free and the output dims can be permuted, so lane c's 8 dims
//    become the c-th row of 8 different 16-dim output blocks and only an
//    in-register 16-bit pack is needed - no LDS transpose.
//  * Every KV load is a buffer load whose resource covers only the slice's
//    valid rows: rows past the descriptor's end read as zero and cost no
//    memory traffic, which masks the unused slots of a request's last page
//    (they may hold NaN).
//  * Two slices are in flight per wave (one computing, one loading): a
//    slice's successor is issued before the slice's math, and a wave's last
//    slice of a descriptor issues nothing.  BF16 runs 8 waves per
//    workgroup, FP8 6: with both slices really in flight, more FP8 waves
//    only added merge work per descriptor and register pressure.
//  * The decode instance drains a bin of many short descriptors one
//    descriptor per wave, with no merge across waves (drain_waves).
//  * A pair served by a single descriptor is finished in place: its
//    normalised output goes straight to `out` in BF16, and a pair without
//    tokens gets zero rows here too.  Only pairs split over several bins use
//    the split buffer.
//  * Merging split pairs (the pages' combine step) can run inside this
//    kernel instead of a second launch: after draining a bin, a workgroup
//    counts one arrival per split pair it served on that pair's counter;
//    the workgroup that completes the count merges the pair's partials in
//    split order.  A pair of more than 16 partials is merged in two levels
//    (groups of f >= 16 consecutive partials, f*f >= count, each merged by
//    the group's last arriver into the group's first slot, then the group
//    results), so no single workgroup reads more than max(16, f) partials
//    per query row.  The eight XCDs keep separate L2 caches, and a
//    device-scope fence would write back or invalidate a whole L2 (hundreds
//    of such fences serialise and stall every workgroup's streaming), so
//    split partials are instead written and read with device-coherent
//    accesses (the sc1 cache policy of agent-scope relaxed atomics, which
//    writes through and reads past the per-XCD caches, at 16 bytes per lane);
//    a workgroup waits for its partial stores to complete before it counts
//    its arrival, once per bin for both of the bin's split pairs (only its
//    first and last descriptor can be split), whose arrivals it counts in
//    parallel.  The last arriver returns each counter to zero.
//  * FP8 KV (OCP e4m3 codes with one fp32 scale per token and KV head): codes
//    are widened to bf16 exactly in registers; the K scale multiplies the
//    score of its token, the V scale is folded into the probability before
//    the bf16 P.V product (sum_t p_t (c_t s_t) = sum_t (p_t s_t) c_t).
//  * Multi-token verification (q_len > 1 query tokens per request, each
//    attending causally up to its own position): the G * q_len query rows of
//    a KV head are the MFMA columns.  Up to 16 columns run the loop above
//    with a per-column causal limit; past 16, every wave keeps one wave
//    state per 16-column tile (up to four) and computes all of them from
//    each slice it loads, so each KV byte is still fetched once per
//    workgroup (see attend_bin).
#include "lse_merge.h"

namespace lbp {
namespace {

// Tunables, fixed at build time per KV format (defaults: the measured best).
#ifndef LBP_BF16_WAVES
#define LBP_BF16_WAVES 8
#endif
#ifndef LBP_FP8_WAVES
#define LBP_FP8_WAVES 6
#endif
#ifndef LBP_BF16_SPLIT_P
#define LBP_BF16_SPLIT_P 1
#endif
#ifndef LBP_FP8Q_WAVES
#define LBP_FP8Q_WAVES 8
#endif
// Multi-token verification: waves of the instances with three or four
// column tiles, and of the two-tile instance per KV format (0: the format's
// own wave count).
#ifndef LBP_TILE_WAVES
#define LBP_TILE_WAVES 4
#endif
#ifndef LBP_BF16_TILE2_WAVES
#define LBP_BF16_TILE2_WAVES 0
#endif
#ifndef LBP_FP8_TILE2_WAVES
#define LBP_FP8_TILE2_WAVES 4
#endif
// Tokens per step of a wave in the tile forms: 16 (1) or 32 (2, one K = 32
// P.V product per pair of 16-token sub-slices).
#ifndef LBP_TILE_SUB
#define LBP_TILE_SUB 2
#endif
// Tile forms: the K scale times the softmax scale once per token (1).
#ifndef LBP_TILE_UNMASKED_LOOP
#define LBP_TILE_UNMASKED_LOOP 1
#endif
#ifndef LBP_TILE_KSFOLD
#define LBP_TILE_KSFOLD 1
#endif
#ifndef LBP_KV_LOAD_AUX
#define LBP_KV_LOAD_AUX 2
#endif
constexpr int kLoadAux = LBP_KV_LOAD_AUX;  // KV and scale loads: 2 = non-temporal (read once, stream)
constexpr int kSlice = 16;
constexpr int kRedRow = kHeadDim + 4;  // padded LDS row (floats) for the merge
// s_waitcnt operand (gfx9 encoding) waiting for vmcnt = 0 only
constexpr int kWaitVmcnt0 = 0x0F70;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw (untyped) buffer, 32-bit data format, as the gfx9 buffer resource
// word 3 requires for offset-addressed loads.
constexpr int kRsrcWord3 = 0x00020000;

__device__ inline rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kRsrcWord3);
}

__device__ inline uint32_t pack_bf16(float lo, float hi) {
  bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// Device-coherent accesses for everything one workgroup writes and another
// merges (the split partials of the in-kernel merge): the cache policy of an
// agent-scope relaxed atomic on gfx950 (sc1: stores write through and loads
// bypass the per-XCD caches), 16 bytes per lane for the partial rows.  They
// go through buffer resources over the split buffer's two sections, which
// are uniform, so each access is one instruction with a per-lane offset.
constexpr int kCoherentAux = 16;   // sc1
struct SplitRsrc {
  rsrc_t o, lse;
};
__device__ inline SplitRsrc split_rsrc(const AttendArgs& a) {
  return SplitRsrc{make_rsrc(a.o_part, a.o_part_bytes), make_rsrc(a.lse_part, a.lse_part_bytes)};
}
// row = descriptor slot * columns + column; c4 = float4 of the row
__device__ inline void store_row_coherent(const SplitRsrc& r, int64_t row, int c4, f32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, v), r.o,
                                         int(row * kHeadDim * 4 + 16 * c4), 0, kCoherentAux);
}
__device__ inline f32x4_t load_row_coherent(const SplitRsrc& r, int64_t row, int c4) {
  return __builtin_bit_cast(
      f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r.o, int(row * kHeadDim * 4 + 16 * c4), 0,
                                                     kCoherentAux));
}
__device__ inline void store_lse_coherent(const SplitRsrc& r, int64_t row, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(int, v), r.lse, int(row * 4), 0,
                                        kCoherentAux);
}
__device__ inline float load_lse_coherent(const SplitRsrc& r, int64_t row) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_raw_buffer_load_b32(r.lse, int(row * 4), 0, kCoherentAux));
}

// Ties a register block to the memory operations issued before it (an empty
// asm statement that clobbers memory and claims to rewrite the block): math
// that reads the block cannot be scheduled above those loads.  The decode
// loop passes the query through it right after issuing the next slice, so
// that slice's loads go out before the current slice's scores instead of
// after them, and two slices stay in flight.
__device__ inline void after_loads(i32x4_t& x) { asm volatile("" : "+v"(x)::"memory"); }
__device__ inline void after_loads(bf16x8_t& x) {
  i32x4_t y = __builtin_bit_cast(i32x4_t, x);
  after_loads(y);
  x = __builtin_bit_cast(bf16x8_t, y);
}

// The four lane groups (lanes n, n + 16, n + 32, n + 48) hold one MFMA
// column.  Their reductions use gfx950's lane swaps instead of a trip
// through the LDS crossbar: swapping a value with a copy of itself across
// the wave's halves (then across neighbouring 16-lane rows) leaves lane l's
// partner l ^ 32 (then l ^ 16) in the pair, in the same order on both
// partners, so all four lanes of a column end with the same result.  Each
// swap is one asm statement (copy, the required wait states, swap) with both
// results as outputs: through the builtin the compiler has merged the two
// results of a swap into one register.
__device__ inline void partners32(float x, float& lo, float& hi) {
  float a = x, b;
  asm("v_mov_b32 %1, %0\n\ts_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1"
      : "+v"(a), "=&v"(b));
  lo = a;   // the value of lane l & 31
  hi = b;   // the value of lane (l & 31) + 32
}
__device__ inline void partners16(float x, float& lo, float& hi) {
  float a = x, b;
  asm("v_mov_b32 %1, %0\n\ts_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1"
      : "+v"(a), "=&v"(b));
  lo = a;   // the value of lane l & ~16
  hi = b;   // the value of lane l | 16
}
// The column reductions over the four lane groups use the swaps above rather
// than cross-lane shuffles through the LDS crossbar: measured faster in every
// KV format.
__device__ inline float wave_max_across_groups(float x) {
  float a, b;
  partners32(x, a, b);
  partners16(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}
__device__ inline float wave_sum_across_groups(float x) {
  float a, b;
  partners32(x, a, b);
  partners16(a + b, a, b);
  return a + b;
}

// ---------------------------------------------------------------------------
// KV formats
// ---------------------------------------------------------------------------

struct SliceRsrc {
  rsrc_t k, v, ks, vs;
};

// Query rows of the query columns: column c is query token c / G, head c % G
// of KV head g's group, at row (r * q_len + c / G) * Hq + g * G + c % G.
// MFMA lane column n of a wave's tile t holds column c = 16 t + n (col0 =
// 16 t below).  The lane's row relative to column 0's, and the
// span of rows the buffer resource covers, depend only on the launch and the
// wave, so they are computed once per kernel (the division stays out of the
// descriptor loop, where it would delay the query loads behind the KV
// loads).  Lanes past the tile's columns get a row past the resource's end
// and read zeros.  With one query token (the non-causal instance, a single
// block) the row is the column itself, which keeps the query offsets equal to
// the K row offsets of the same lanes.
struct QLane {
  int row;    // this lane's row relative to column 0's, or past `rows` (reads 0)
  int rows;   // rows the resource spans
};
template <bool kMultiToken>
__device__ inline QLane q_lane(const AttendArgs& a, int n, int col0, int block_valid) {
  QLane q;
  if constexpr (kMultiToken) {
    const int c = col0 + n;
    q.rows = (a.q_len - 1) * a.num_q_heads + a.group;
    q.row = n < block_valid ? (c / a.group) * a.num_q_heads + c % a.group : q.rows;
  } else {
    q.rows = a.group;
    q.row = n;
  }
  return q;
}
__device__ inline int64_t q_base_row(const AttendArgs& a, int g, int r) {
  return int64_t(r) * a.q_len * a.num_q_heads + int64_t(g) * a.group;
}

// BF16 query columns as the MFMA B operand, in the dim order of format Kv.
template <class Kv>
__device__ inline void load_q_bf16(bf16x8_t* qb, const AttendArgs& a, const QLane& ql, int g,
                                   int r, int grp) {
  const rsrc_t qr = make_rsrc(static_cast<const char*>(a.q) + q_base_row(a, g, r) * kHeadDim * 2,
                              ql.rows * kHeadDim * 2);
#pragma unroll
  for (int s = 0; s < 4; ++s)
    qb[s] = __builtin_bit_cast(
        bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(
                      qr, ql.row * kHeadDim * 2 + Kv::q_offset(0, grp, s), 0, 0));
}

struct Bf16Kv {
  static constexpr int kRowBytes = kHeadDim * 2;
  static constexpr bool kScaled = false;
  static constexpr bool kSplitP = LBP_BF16_SPLIT_P;   // P.V with P as BF16 hi + lo
  // two-tile verification instance: its wave count (0: kWaves)
  static constexpr int kTile2Waves = LBP_BF16_TILE2_WAVES;
  static constexpr int kWaves = LBP_BF16_WAVES;    // waves per workgroup
  struct Buf {
    i32x4_t k[4];   // K A-operand, one per 32-dim k-step
    i32x4_t v[4];   // V rows 4*grp+i, dims [8c, 8c+8)
  };
  // Q B-operand for k-step s: dims [32s + 8grp, +8) of head n.
  __device__ static int q_offset(int n, int grp, int s) { return n * 256 + 64 * s + 16 * grp; }
  struct Q {
    bf16x8_t v[4];
  };
  __device__ static void load_q(Q& q, const AttendArgs& a, const QLane& ql, int g, int r,
                                int grp) {
    load_q_bf16<Bf16Kv>(q.v, a, ql, g, r, grp);
  }
  __device__ static float score_scale(const Q&, float scale_log2) { return scale_log2; }
  __device__ static void after_loads(Q& q) {
#pragma unroll
    for (int k = 0; k < 4; ++k) lbp::after_loads(q.v[k]);
  }

  __device__ static void issue(Buf& b, const SliceRsrc& rs, int lane) {
    const int m = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      b.k[s] = __builtin_amdgcn_raw_buffer_load_b128(rs.k, m * kRowBytes + 64 * s + 16 * grp, 0, kLoadAux);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      b.v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs.v, (4 * grp + i) * kRowBytes + 16 * m, 0, kLoadAux);
  }

  // (B: any slice type holding the K operand as member k)
  template <class B>
  __device__ static f32x4_t scores(const B& b, const Q& q) {
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, b.k[k]), q.v[k], s,
                                                  0, 0, 0);
    return s;
  }
  // k-step k of the score product (K operand of the step, the query's)
  __device__ static bf16x8_t k_step(const Buf& b, int k) { return __builtin_bit_cast(bf16x8_t, b.k[k]); }
  __device__ static f32x4_t score_step(bf16x8_t kop, const Q& q, int k, f32x4_t s) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, q.v[k], s, 0, 0, 0);
  }
  __device__ static f32x4_t k_scales(const Buf&) { return f32x4_t{1.f, 1.f, 1.f, 1.f}; }
  __device__ static f32x4_t v_scales(const Buf&) { return f32x4_t{1.f, 1.f, 1.f, 1.f}; }

  // A operand of output block mb (dims 8c + mb) over the slice's 16 tokens.
  __device__ static i16x4_t v_operand(const Buf& b, int mb) {
    const int w = mb >> 1;
    uint32_t x0 = b.v[0][w], x1 = b.v[1][w], x2 = b.v[2][w], x3 = b.v[3][w];
    uint32_t lo, hi;
    if (mb & 1) {
      lo = (x0 >> 16) | (x1 & 0xFFFF0000u);
      hi = (x2 >> 16) | (x3 & 0xFFFF0000u);
    } else {
      lo = (x0 & 0xFFFFu) | (x1 << 16);
      hi = (x2 & 0xFFFFu) | (x3 << 16);
    }
    i32x2_t r = {int(lo), int(hi)};
    return __builtin_bit_cast(i16x4_t, r);
  }
};

struct Fp8Kv {
  static constexpr int kRowBytes = kHeadDim;
  static constexpr bool kScaled = true;
  // the FP8 tolerance leaves room for P in plain BF16, and this format needs
  // its issue slots for the code widening
  static constexpr bool kSplitP = false;
  // waves per workgroup: FP8 moves half the bytes per token, but 6 waves with
  // two slices each keep enough loads in flight, and fewer waves make each
  // descriptor's merge cheaper
  static constexpr int kWaves = LBP_FP8_WAVES;
  // two-tile verification instance: one wave per SIMD, 32-token spans (the
  // widening leaves a two-wave instance short of registers for both tiles)
  static constexpr int kTile2Waves = LBP_FP8_TILE2_WAVES;
  struct Buf {
    i32x4_t k[2];   // 32 codes: dims [32grp, 32grp + 32) of token m
    i32x2_t v[4];   // 8 codes: dims [8c, 8c+8) of token 4grp+i
    i32x4_t ks;     // k scales of tokens 4grp .. 4grp+3
    i32x4_t vs;     // v scales of tokens 4grp .. 4grp+3
  };
  // Q B-operand for k-step s: dims [32grp + 8s, +8) of head n.
  __device__ static int q_offset(int n, int grp, int s) { return n * 256 + 64 * grp + 16 * s; }
  struct Q {
    bf16x8_t v[4];
  };
  __device__ static void load_q(Q& q, const AttendArgs& a, const QLane& ql, int g, int r,
                                int grp) {
    load_q_bf16<Fp8Kv>(q.v, a, ql, g, r, grp);
  }
  __device__ static float score_scale(const Q&, float scale_log2) { return scale_log2; }
  __device__ static void after_loads(Q& q) {
#pragma unroll
    for (int k = 0; k < 4; ++k) lbp::after_loads(q.v[k]);
  }

  __device__ static void issue(Buf& b, const SliceRsrc& rs, int lane) {
    const int m = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      b.k[h] = __builtin_amdgcn_raw_buffer_load_b128(rs.k, m * kRowBytes + 32 * grp + 16 * h, 0, kLoadAux);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      b.v[i] = __builtin_amdgcn_raw_buffer_load_b64(rs.v, (4 * grp + i) * kRowBytes + 8 * m, 0, kLoadAux);
    b.ks = __builtin_amdgcn_raw_buffer_load_b128(rs.ks, 16 * grp, 0, kLoadAux);
    b.vs = __builtin_amdgcn_raw_buffer_load_b128(rs.vs, 16 * grp, 0, kLoadAux);
  }

  // Two e4m3 codes (the low or high 16-bit word of `codes`) to two bf16, exactly.
  template <bool kHiWord>
  __device__ static uint32_t widen2(uint32_t codes) {
    return __builtin_bit_cast(uint32_t,
                              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(int(codes), 1.0f, kHiWord));
  }

  // K operand of k-step k as eight BF16 values (exact)
  template <class B>
  __device__ static i32x4_t k_bf16(const B& b, int k) {
    uint32_t c0 = b.k[k >> 1][2 * (k & 1)], c1 = b.k[k >> 1][2 * (k & 1) + 1];
    return i32x4_t{int(widen2<false>(c0)), int(widen2<true>(c0)), int(widen2<false>(c1)),
                   int(widen2<true>(c1))};
  }

  template <class B>
  __device__ static f32x4_t scores(const B& b, const Q& q) {
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, k_bf16(b, k)),
                                                  q.v[k], s, 0, 0, 0);
    return s;
  }
  __device__ static bf16x8_t k_step(const Buf& b, int k) {
    return __builtin_bit_cast(bf16x8_t, k_bf16(b, k));
  }
  __device__ static f32x4_t score_step(bf16x8_t kop, const Q& q, int k, f32x4_t s) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, q.v[k], s, 0, 0, 0);
  }
  __device__ static f32x4_t k_scales(const Buf& b) { return __builtin_bit_cast(f32x4_t, b.ks); }
  __device__ static f32x4_t v_scales(const Buf& b) { return __builtin_bit_cast(f32x4_t, b.vs); }

  __device__ static i16x4_t v_operand(const Buf& b, int mb) {
    const int h = mb >> 2;           // which dword of the 8 codes
    const int k = mb & 3;            // byte inside it
    // bytes {t0.bk, t1.bk, t0.bk+1, t1.bk+1} for the token pairs (0,1), (2,3)
    const uint32_t sel = (k < 2) ? 0x05010400u : 0x07030602u;
    uint32_t p01 = __builtin_amdgcn_perm(uint32_t(b.v[1][h]), uint32_t(b.v[0][h]), sel);
    uint32_t p23 = __builtin_amdgcn_perm(uint32_t(b.v[3][h]), uint32_t(b.v[2][h]), sel);
    i32x2_t r;
    if (k & 1)
      r = i32x2_t{int(widen2<true>(p01)), int(widen2<true>(p23))};
    else
      r = i32x2_t{int(widen2<false>(p01)), int(widen2<false>(p23))};
    return __builtin_bit_cast(i16x4_t, r);
  }
};


// FP8 KV with an FP8 query (OCP e4m3 codes and one fp32 scale per request and
// query head, as the fused attention prologue emits them): the score product
// runs on the fp8 x fp8 MFMA straight from the K and Q codes, with no
// widening; the Q scale joins the softmax scale per head.  V and the
// probabilities take the FP8 KV path above.
struct Fp8KvQ8 : Fp8Kv {
  static constexpr int kWaves = LBP_FP8Q_WAVES;
  struct Q {
    i32x4_t c[2];   // codes of dims [32grp, 32grp + 32) of head n
    float scale;    // the head's Q scale (0 for columns past the group)
  };
  __device__ static void load_q(Q& q, const AttendArgs& a, const QLane& ql, int g, int r,
                                int grp) {
    const int64_t base = q_base_row(a, g, r);
    const rsrc_t qr = make_rsrc(static_cast<const char*>(a.q) + base * kHeadDim,
                                ql.rows * kHeadDim);
    const rsrc_t sr = make_rsrc(a.q_scale + base, ql.rows * 4);
#pragma unroll
    for (int h = 0; h < 2; ++h)
      q.c[h] = __builtin_amdgcn_raw_buffer_load_b128(qr, ql.row * kHeadDim + 32 * grp + 16 * h,
                                                     0, 0);
    q.scale = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, 4 * ql.row, 0, 0));
  }
  __device__ static float score_scale(const Q& q, float scale_log2) { return q.scale * scale_log2; }
  __device__ static void after_loads(Q& q) {
    lbp::after_loads(q.c[0]);
    lbp::after_loads(q.c[1]);
  }

  // 8 codes (one k-step of 32 dims split over the four lane groups) as an
  // fp8 MFMA operand.
  __device__ static long codes8(const i32x4_t* c, int k) {
    typedef long i64x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(i64x2_t, c[k >> 1])[k & 1];
  }
  template <class B>
  __device__ static f32x4_t scores(const B& b, const Q& q) {
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k)
      s = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(codes8(b.k, k), codes8(q.c, k), s, 0, 0, 0);
    return s;
  }
  __device__ static long k_step(const Buf& b, int k) { return codes8(b.k, k); }
  __device__ static f32x4_t score_step(long kop, const Q& q, int k, f32x4_t s) {
    return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(kop, codes8(q.c, k), s, 0, 0, 0);
  }
};

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------

// Number of slices a wave takes from [t, e) when its slices start at t and
// advance by `stride` tokens.
__device__ inline int wave_slices(int t, int e, int stride) {
  return t < e ? (e - t + stride - 1) / stride : 0;
}

// The read-only tables (page table, descriptors, pair counts, bin offsets)
// reach the kernel as separate `const __restrict__` parameters: proven
// unaliased with the kernel's stores, their wave-uniform reads compile to
// scalar loads, which complete on the scalar counter.  Looking up the next
// slice's page then never waits for the KV loads still in flight (vector
// loads complete in order, so a vector load of the page index would).
// The physical page of the slice at token tok of request r (its last page's
// for a slice past the end e, which loads nothing).
__device__ inline int page_of(const AttendArgs& a, const int32_t* __restrict__ pt, int r, int tok,
                              int e) {
  const int pidx = (tok < e ? tok : e - 1) >> 6;
  return pt[int64_t(r) * a.page_table_stride + pidx];
}
template <class Kv>
__device__ inline SliceRsrc slice_rsrc_at(const AttendArgs& a, int g, int tok, int e, int page) {
  const bool valid = tok < e;
  const int nvalid = valid ? min(kSlice, e - tok) : 0;
  const int64_t row = (int64_t(page) * a.num_kv_heads + g) * kPageTokens + (tok & (kPageTokens - 1));
  SliceRsrc rs;
  rs.k = make_rsrc(static_cast<const char*>(a.k_cache) + row * Kv::kRowBytes, nvalid * Kv::kRowBytes);
  rs.v = make_rsrc(static_cast<const char*>(a.v_cache) + row * Kv::kRowBytes, nvalid * Kv::kRowBytes);
  if constexpr (Kv::kScaled) {
    rs.ks = make_rsrc(a.k_scale + row, nvalid * 4);
    rs.vs = make_rsrc(a.v_scale + row, nvalid * 4);
  } else {
    rs.ks = rs.k;
    rs.vs = rs.v;
  }
  return rs;
}
template <class Kv>
__device__ inline SliceRsrc slice_rsrc(const AttendArgs& a, const int32_t* __restrict__ pt, int g,
                                       int r, int tok, int e) {
  return slice_rsrc_at<Kv>(a, g, tok, e, page_of(a, pt, r, tok, e));
}

struct WaveState {
  float m;          // running max of log2-scaled scores (per head n = lane & 15)
  float l;          // this lane's share of the running sum
  f32x4_t acc[8];   // O^T blocks: lane (grp, n) holds dims 32grp + 8j + mb
};

// One slice into one wave state (decode, and verification up to 16
// columns).  lim: this lane's column sees tokens < lim (its causal limit in
// multi-token verification, kCausal only).  A column with no visible token
// so far keeps an empty state (m = -inf, l = 0, acc = 0).
template <class Kv, bool kCausal>
__device__ inline void consume(WaveState& st, const typename Kv::Buf& b, const typename Kv::Q& q,
                               int tok, int e, float scale_log2, int grp, int lim) {
  f32x4_t s = Kv::scores(b, q);
  f32x4_t ks = Kv::k_scales(b);
  f32x4_t vs = Kv::v_scales(b);
  float x[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    x[j] = (tok + 4 * grp + j < (kCausal ? min(e, lim) : e)) ? s[j] * ks[j] * scale_log2
                                                             : -INFINITY;
  float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
  mx = wave_max_across_groups(mx);
  const float m_new = fmaxf(st.m, mx);
  // without a causal limit every slice has a visible token in every column,
  // so the running max is finite after the first one
  const float ref = kCausal ? finite_or_zero(m_new) : m_new;
  {
    const float alpha = __builtin_amdgcn_exp2f(st.m - ref);
    st.l *= alpha;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) st.acc[mb] *= alpha;
  }
  st.m = m_new;
  // BF16 KV: P enters the P.V product as a BF16 pair (below), which the
  // HBM-bound decode loop pays nothing for.  The FP8 formats fold the V
  // scale into P and keep one BF16 P with l from the unrounded values.
  float p[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) p[j] = __builtin_amdgcn_exp2f(x[j] - ref);
  st.l += (p[0] + p[1]) + (p[2] + p[3]);
  if constexpr (Kv::kSplitP) {
    const float pv[4] = {p[0] * vs[0], p[1] * vs[1], p[2] * vs[2], p[3] * vs[3]};
    i32x2_t pb2 = {int(pack_bf16(pv[0], pv[1])), int(pack_bf16(pv[2], pv[3]))};
    const i16x4_t pb = __builtin_bit_cast(i16x4_t, pb2);
    // P as a BF16 pair hi + lo (lo = the rounding residual of hi): the P.V
    // product then carries P to ~2^-17 instead of BF16's 2^-9, at the cost
    // of a second MFMA per output block, of which this HBM-bound kernel has
    // plenty to spare
    const uint32_t h01 = uint32_t(pb2[0]), h23 = uint32_t(pb2[1]);
    const float r0 = pv[0] - __builtin_bit_cast(float, h01 << 16);
    const float r1 = pv[1] - __builtin_bit_cast(float, h01 & 0xFFFF0000u);
    const float r2 = pv[2] - __builtin_bit_cast(float, h23 << 16);
    const float r3 = pv[3] - __builtin_bit_cast(float, h23 & 0xFFFF0000u);
    i32x2_t lo2 = {int(pack_bf16(r0, r1)), int(pack_bf16(r2, r3))};
    const i16x4_t pl = __builtin_bit_cast(i16x4_t, lo2);
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const i16x4_t vop = Kv::v_operand(b, mb);
      st.acc[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, pb, st.acc[mb], 0, 0, 0);
      st.acc[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vop, pl, st.acc[mb], 0, 0, 0);
    }
  } else {
    i32x2_t pb2 = {int(pack_bf16(p[0] * vs[0], p[1] * vs[1])),
                   int(pack_bf16(p[2] * vs[2], p[3] * vs[3]))};
    const i16x4_t pb = __builtin_bit_cast(i16x4_t, pb2);
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
      st.acc[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(Kv::v_operand(b, mb), pb,
                                                              st.acc[mb], 0, 0, 0);
  }
}

// consume for kNB column tiles of one slice (the causal tile forms), in
// phases across the tiles: every tile's scores and running max first, then a
// single rescale of all tiles when any lane of any tile saw its maximum grow
// (a tile that did not grow is multiplied by exactly 1, so the results are
// those of a rescale per tile, bit for bit), then every tile's probabilities
// and P.V products.  The tiles' chains are independent, and with one branch
// per slice instead of one per tile the scheduler can interleave them, which
// a wave alone on its SIMD needs to hide the MFMA and transcendental
// latencies.  Bound by their math rather than by HBM, these forms take P as
// one BF16 value instead of consume's BF16 pair; for BF16 KV they sum the same
// rounded values into l, so the output is an exact convex combination of the
// V rows under the rounded weights, whose error scales with |v - o| rather
// than |v| (a row with one dominant token stays exact).  The FP8 formats
// keep l from the unrounded values, as in consume.
// kSub = 2: the slice is 32 tokens, two 16-token sub-slices b[0] and b[1],
// whose P.V is a single MFMA with K = 32 per output block.
template <class Kv, bool kCausal, int kNB, int kSub, bool kMask = true>
__device__ inline void consume_tiles(WaveState (&st)[kNB], const typename Kv::Buf (&b)[kSub],
                                     const typename Kv::Q (&q)[kNB], int tok, int e,
                                     const float (&scale_log2)[kNB], int grp,
                                     const int (&lim)[kNB]) {
  static_assert(kSub == 1 || kSub == 2, "one or two 16-token sub-slices");
  f32x4_t ks[kSub], vs[kSub];
#pragma unroll
  for (int u = 0; u < kSub; ++u) {
    ks[u] = Kv::k_scales(b[u]);
    vs[u] = Kv::v_scales(b[u]);
  }
  // the score products with the k-step outermost: each K operand (for FP8
  // the widened codes) serves the kNB tiles' independent MFMAs at once and
  // is dead after them
  f32x4_t scs[kNB][kSub];
#pragma unroll
  for (int u = 0; u < kSub; ++u) {
#pragma unroll
    for (int t = 0; t < kNB; ++t) scs[t][u] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const auto kop = Kv::k_step(b[u], k);
#pragma unroll
      for (int t = 0; t < kNB; ++t) scs[t][u] = Kv::score_step(kop, q[t], k, scs[t][u]);
    }
  }
  float x[kNB][kSub][4];
  float m_new[kNB];
  bool grew = false;
#pragma unroll
  for (int t = 0; t < kNB; ++t) {
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < kSub; ++u) {
      const f32x4_t sc = scs[t][u];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float v = LBP_TILE_KSFOLD ? sc[j] * (ks[u][j] * scale_log2[t])
                                        : sc[j] * ks[u][j] * scale_log2[t];
        x[t][u][j] = !kMask || tok + kSlice * u + 4 * grp + j < (kCausal ? min(e, lim[t]) : e)
                         ? v
                         : -INFINITY;
      }
      mx = fmaxf(mx, fmaxf(fmaxf(x[t][u][0], x[t][u][1]), fmaxf(x[t][u][2], x[t][u][3])));
    }
    mx = wave_max_across_groups(mx);
    m_new[t] = fmaxf(st[t].m, mx);
    grew = grew || m_new[t] > st[t].m;
  }
  if (__ballot(grew) != 0) {
    asm volatile("");   // keeps the skip a branch (see consume)
#pragma unroll
    for (int t = 0; t < kNB; ++t) {
      const float ref = kCausal ? finite_or_zero(m_new[t]) : m_new[t];
      const float alpha = __builtin_amdgcn_exp2f(st[t].m - ref);
      st[t].l *= alpha;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) st[t].acc[mb] *= alpha;
    }
  }
  constexpr bool kRoundedSum = Kv::kSplitP;
  // every tile's P first, then the P.V products with the output block
  // outermost: each V operand (for FP8 the widened codes) serves the kNB
  // tiles' independent MFMAs at once and is dead after them
  i32x2_t pbs[kNB][kSub];
#pragma unroll
  for (int t = 0; t < kNB; ++t) {
    st[t].m = m_new[t];
    const float ref = kCausal ? finite_or_zero(m_new[t]) : m_new[t];
    i32x2_t (&pb2)[kSub] = pbs[t];
#pragma unroll
    for (int u = 0; u < kSub; ++u) {
      float p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) p[j] = __builtin_amdgcn_exp2f(x[t][u][j] - ref);
      if constexpr (!kRoundedSum) st[t].l += (p[0] + p[1]) + (p[2] + p[3]);
      pb2[u] = i32x2_t{int(pack_bf16(p[0] * vs[u][0], p[1] * vs[u][1])),
                       int(pack_bf16(p[2] * vs[u][2], p[3] * vs[u][3]))};
      if constexpr (kRoundedSum) {
        const uint32_t h01 = uint32_t(pb2[u][0]), h23 = uint32_t(pb2[u][1]);
        st[t].l += (__builtin_bit_cast(float, h01 << 16) +
                    __builtin_bit_cast(float, h01 & 0xFFFF0000u)) +
                   (__builtin_bit_cast(float, h23 << 16) +
                    __builtin_bit_cast(float, h23 & 0xFFFF0000u));
      }
    }
  }
#pragma unroll
  for (int mb = 0; mb < 8; ++mb) {
    if constexpr (kSub == 1) {
      const i16x4_t vop = Kv::v_operand(b[0], mb);
#pragma unroll
      for (int t = 0; t < kNB; ++t)
        st[t].acc[mb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
            vop, __builtin_bit_cast(i16x4_t, pbs[t][0]), st[t].acc[mb], 0, 0, 0);
    } else {
      // one K = 32 product over both sub-slices: contraction index 8 grp + i
      // is token 4 grp + (i mod 4) of sub-slice i / 4, in P and in V alike
      const i32x2_t v0 = __builtin_bit_cast(i32x2_t, Kv::v_operand(b[0], mb));
      const i32x2_t v1 = __builtin_bit_cast(i32x2_t, Kv::v_operand(b[1], mb));
      const i32x4_t vw = {v0[0], v0[1], v1[0], v1[1]};
      const bf16x8_t vop = __builtin_bit_cast(bf16x8_t, vw);
#pragma unroll
      for (int t = 0; t < kNB; ++t) {
        const i32x4_t pw = {pbs[t][0][0], pbs[t][0][1], pbs[t][1][0], pbs[t][1][1]};
        st[t].acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, __builtin_bit_cast(bf16x8_t, pw),
                                                                st[t].acc[mb], 0, 0, 0);
      }
    }
  }
}

// The wave count of an instance: the format's own, or kTileW for a causal
// instance with several column tiles.
template <class Kv, int kTileW = 0>
constexpr int waves_of() {
  return kTileW > 0 ? kTileW : Kv::kWaves;
}
constexpr int kTileWaves = LBP_TILE_WAVES;   // instances with three or four tiles

// The loads of one wave step: one 16-token slice, or kSub consecutive ones
// (the tile forms' 32-token spans).
template <class Kv, int kSub>
struct SpanOf {
  typename Kv::Buf s[kSub];
};
template <class Kv, int kSub>
using SpanBuf = std::conditional_t<kSub == 1, typename Kv::Buf, SpanOf<Kv, kSub>>;

// Drains a bin of many short descriptors, one descriptor per wave.
//
// attend_bin ends every descriptor with a merge of all waves' states through
// LDS between two workgroup barriers, and the next descriptor's first loads
// wait for this one's last: about 1.1 us per boundary, more than a 64-token
// tile of streaming.  Where short requests pile up (the plan fills bins in
// request order, so a bin can hold many pairs of one or two tiles) the
// boundaries dominate.  Here wave w instead takes the bin's descriptors
// w, w + W, ... and drains each one alone, its 16-token slices in order
// with two in flight, then writes its result straight from its registers:
// the normalised row of a pair with one descriptor, else the partial row and
// its log-sum-exp for the combine kernel.  No LDS, no barrier, and the waves'
// descriptor chains overlap.  Decode only (one column tile, no causal
// limit, no in-kernel merge).
template <class Kv>
__device__ inline void drain_waves(const AttendArgs& a, const int32_t* __restrict__ pt,
                                   const int4* __restrict__ descs,
                                   const int32_t* __restrict__ pair_count, int d_begin, int d_end,
                                   int wave, int lane) {
  constexpr int kWaves = Kv::kWaves;
  int d = d_begin + wave;
  if (d >= d_end) return;
  const int n = lane & 15, grp = lane >> 4;
  const int C = a.ncols;   // = G: one query token
  const QLane ql = q_lane<false>(a, n, 0, C);
  int4 ds = descs[d];
  typename Kv::Q qb;
  typename Kv::Buf buf[2];
  Kv::load_q(qb, a, ql, ds.x, ds.y, grp);
  Kv::issue(buf[0], slice_rsrc<Kv>(a, pt, ds.x, ds.y, ds.z, ds.w), lane);
  for (; d < d_end; d += kWaves) {
    const int g = ds.x, r = ds.y, t_end = ds.w;
    const bool single = pair_count[g * a.batch + r] == 1;
    const bool has_next = d + kWaves < d_end;
    const int4 dn = descs[has_next ? d + kWaves : d];
    const int next_page = page_of(a, pt, dn.y, dn.z, dn.w);
    WaveState st;
    st.m = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) st.acc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // the descriptor's ns >= 1 slices, the first in (or loading into)
    // buf[0]; as in attend_bin, a slice with a successor issues it before
    // its own math, and one code path computes every last slice
    int tok = ds.z;
    const int ns = wave_slices(tok, t_end, kSlice);
    const float sc = Kv::score_scale(qb, a.scale_log2);
    auto step_on = [&](const typename Kv::Buf& cur, typename Kv::Buf& nxt) {
      Kv::issue(nxt, slice_rsrc<Kv>(a, pt, g, r, tok + kSlice, t_end), lane);
      Kv::after_loads(qb);
      consume<Kv, false>(st, cur, qb, tok, t_end, sc, grp, INT_MAX);
      tok += kSlice;
    };
    for (int i = (ns - 1) >> 1; i > 0; --i) {
      step_on(buf[0], buf[1]);
      step_on(buf[1], buf[0]);
    }
    if ((ns & 1) == 0) {
      step_on(buf[0], buf[1]);
      buf[0] = buf[1];
    }
    consume<Kv, false>(st, buf[0], qb, tok, t_end, sc, grp, INT_MAX);
    // this wave's next descriptor: query and first slice, before the stores
    if (has_next) {
      Kv::load_q(qb, a, ql, dn.x, dn.y, grp);
      Kv::issue(buf[0], slice_rsrc_at<Kv>(a, dn.x, dn.z, dn.w, next_page), lane);
    }
    // lane (grp, n) holds dims 32 grp + 8 j + mb of column n: per j, the
    // float4s 8 grp + 2 j (mb 0-3) and 8 grp + 2 j + 1 (mb 4-7)
    const float L = wave_sum_across_groups(st.l);
    const float inv = 1.f / L;
    if (n < C) {
      auto half = [&](int j, int h) {
        return f32x4_t{st.acc[4 * h][j], st.acc[4 * h + 1][j], st.acc[4 * h + 2][j],
                       st.acc[4 * h + 3][j]} * inv;
      };
      if (single) {
        const int64_t row = int64_t(r) * a.num_q_heads + int64_t(g) * C + n;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int h = 0; h < 2; ++h) store_bf16x4(a.out, row, 8 * grp + 2 * j + h, half(j, h));
      } else {
        const int64_t e = int64_t(d) * C + n;
        f32x4_t* po = reinterpret_cast<f32x4_t*>(a.o_part + e * kHeadDim) + 8 * grp;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int h = 0; h < 2; ++h) po[2 * j + h] = half(j, h);
        if (grp == 0) a.lse_part[e] = st.m + __builtin_amdgcn_logf(L);
      }
    }
    ds = dn;
  }
}

// Drains one bin: every descriptor in it, in order.
//
// Slice i of a descriptor goes to wave i % kWaves; each wave keeps two
// slices in flight (one computing, one loading).  As soon as a wave has
// consumed its last slice of descriptor d it issues its first slice of
// d + 1 and d + 1's query group, before the cross-wave merge of d, so their
// latency overlaps the merge and the wait for the slowest wave instead of
// following them.
//
// kNB: 16-column MFMA tiles per wave (1 for decode and up to 16 query
// columns; 2, 3 or 4 for 17-64 columns in multi-token verification: every
// wave keeps a wave state per tile and computes all of them from each slice
// it loads, so every KV byte is still fetched once per workgroup).  kTileW:
// the tile form's wave count (0: the format's own).  With one wave per SIMD
// the register file has room for 32-token spans (two slices per step).
template <class Kv, bool kCausal, int kNB, int kTileW, bool kFuse>
__device__ inline void attend_bin(const AttendArgs& a, const int32_t* __restrict__ pt,
                                  const int4* __restrict__ descs,
                                  const int32_t* __restrict__ pair_count,
                                  const int32_t* __restrict__ bin_offset,
                                  const int4* __restrict__ bin_first,
                                  const int32_t* __restrict__ pair_first, float* smem, int bin) {
  constexpr int kWaves = waves_of<Kv, kTileW>();
  constexpr int kThreads = kWaves * 64;
  static_assert(kNB == 1 || (kNB <= 4 && kCausal),
                "several column tiles per wave: causal form only");
  static_assert(kTileW == 0 || kNB > 1, "a wave count of its own: tile forms only");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;         // MFMA column of this lane within its block
  const int grp = lane >> 4;
  const int G = a.group;
  const int C = a.ncols;           // G * q_len: every wave computes all C <= 16 kNB
  // the tile forms with one wave per SIMD (512 registers) step by spans of
  // kSub 16-token sub-slices; at two waves per SIMD the second sub-slice's
  // registers do not fit
  constexpr int kSub = kNB > 1 && kWaves <= 4 ? LBP_TILE_SUB : 1;
  constexpr int kSpan = kSlice * kSub;
  constexpr int step = kWaves * kSpan;                 // a wave's stride in tokens
  using SBuf = SpanBuf<Kv, kSub>;
  // per wave in LDS for the merge: m and l of 16 kNB columns, then the rows
  constexpr int kRedHead = 32 * kNB;
  const int red_stride = kRedHead + C * kRedRow;
  // tile t's columns: [16 t, + tile_cols(t))
  auto tile_cols = [&](int t) { return kNB == 1 ? C : min(16, C - 16 * t); };
  float* red = smem + wave * red_stride;
  // range, first descriptor and the pages of its first two tiles are
  // independent loads: one round trip, after which the first KV loads can
  // issue without a page-table lookup
  const int d_begin = bin_offset[bin];
  const int d_end = bin_offset[bin + 1];
  int4 ds = bin_first[2 * bin];
  const int4 first_pages = bin_first[2 * bin + 1];
  asm volatile("" ::"s"(ds.x), "s"(ds.y), "s"(ds.z), "s"(ds.w), "s"(first_pages.x),
               "s"(first_pages.y));   // keep the loads above the exit
  if (d_begin >= d_end) return;
  if constexpr (!kCausal && kNB == 1 && !kFuse) {
    // at least three descriptors of at most two tiles on average (every
    // bin but the last holds exactly `budget` tiles, the last fewer): one
    // descriptor per wave.  Marked unlikely so that the compiler places
    // drain_waves after the loop below instead of between this test and it,
    // which costs short launches less
    const int budget = bin_offset[kHdrBudget - kHdrWords];
    if (__builtin_expect(d_end - d_begin >= 3 && budget <= 2 * (d_end - d_begin), 0)) {
      drain_waves<Kv>(a, pt, descs, pair_count, d_begin, d_end, wave, lane);
      return;
    }
  }

  QLane ql[kNB];
  typename Kv::Q qb[kNB];
  SBuf buf[2];
  // the span at token t of KV head gq, whose page (tokens t and t + 16 share
  // it: spans start at multiples of 32) is `page`
  auto issue_span = [&](SBuf& b, int gq, int t, int e, int page) {
    if constexpr (kSub == 1) {
      Kv::issue(b, slice_rsrc_at<Kv>(a, gq, t, e, page), lane);
    } else {
#pragma unroll
      for (int u = 0; u < kSub; ++u)
        Kv::issue(b.s[u], slice_rsrc_at<Kv>(a, gq, t + kSlice * u, e, page), lane);
    }
  };
  if constexpr (kNB == 1) {
    // (spelled out: the loop form below, though equivalent, made the
    // compiler schedule the decode instance differently, and slower)
    ql[0] = q_lane<kCausal>(a, n, 0, C);
    Kv::load_q(qb[0], a, ql[0], ds.x, ds.y, grp);
  } else {
#pragma unroll
    for (int t = 0; t < kNB; ++t) {
      ql[t] = q_lane<kCausal>(a, n, 16 * t, tile_cols(t));
      Kv::load_q(qb[t], a, ql[t], ds.x, ds.y, grp);
    }
  }
  {
    // a wave's first span starts in the descriptor's first or second tile
    // (or, past a short descriptor's end, loads nothing from its last one):
    // the page page_of would look up
    static_assert((kWaves - 1) * kSpan < 2 * kPageTokens, "first spans within two tiles");
    const int t0 = ds.z + wave * kSpan;
    issue_span(buf[0], ds.x, t0, ds.w, wave * kSpan < kPageTokens ? first_pages.x : first_pages.y);
  }

  for (int d = d_begin; d < d_end; ++d) {
    const int g = ds.x, r = ds.y, t_begin = ds.z, t_end = ds.w;
    const int p = g * a.batch + r;
    const bool single = pair_count[p] == 1;
    const bool has_next = d + 1 < d_end;
    const int4 dn = descs[has_next ? d + 1 : d];
    // the next descriptor's first slice of this wave and its page, looked up
    // now so that the lookup completes during this descriptor's loop instead
    // of delaying the prefetch after it
    const int next_tok = (has_next ? dn.z : dn.w) + wave * kSpan;
    const int next_page = page_of(a, pt, dn.y, next_tok, dn.w);
    // causal limit of this lane's column in multi-token verification: query
    // token j of the request sits at position L - q_len + j, L being the
    // end of the pair's last descriptor
    int lim[kNB];
    WaveState st[kNB];
#pragma unroll
    for (int t = 0; t < kNB; ++t) {
      lim[t] = INT_MAX;
      if constexpr (kCausal) {
        const int L = descs[pair_first[p] + pair_count[p] - 1].w;
        lim[t] = L - a.q_len + 1 + (16 * t + n) / G;
      }
      st[t].m = -INFINITY;
      st[t].l = 0.f;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) st[t].acc[mb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // The wave's n slices (spans) of the descriptor, the first already in
    // (or loading into) buf[0]; a slice past t_end loads nothing.  Each one
    // that has a successor issues the successor's loads and then computes,
    // with both in flight; the last one issues nothing (the next
    // descriptor's loads follow the loop; a load past the end, though it
    // moves no data, costs as much issue and queue time as a real one).
    // Whole trips of two steps, then for even n one more step and a copy of
    // the last slice from buf[1] to buf[0] (which waits for it), so a single
    // code path computes every last slice: with one such path per parity the
    // compiler kept two copies of the wave state.  The loop has one exit and
    // every path to a step has the same loads outstanding, so the compiler's
    // wait counts stay exact.
    int tok = t_begin + wave * kSpan;
    const int ns = wave_slices(tok, t_end, step);
    // (one tile spelled out, as in the query setup above)
    const float sc0 = Kv::score_scale(qb[0], a.scale_log2);
    // kMask: the per-token mask of the descriptor's end and the causal
    // limits.  In the tile forms only a wave's last span can need it: the
    // spans before it end at least step - kSpan tokens before the
    // descriptor's end, and no query token's limit lies more than
    // q_len - 1 <= C - 1 tokens before the pair's end.
    static_assert(kNB == 1 || step - kSpan + 2 > 16 * kNB, "unmasked spans must be whole");
    auto compute = [&](const SBuf& cur, auto mask) {
      if constexpr (kNB == 1) {
        consume<Kv, kCausal>(st[0], cur, qb[0], tok, t_end, sc0, grp, lim[0]);
      } else {
        constexpr bool kMask = decltype(mask)::value || !LBP_TILE_UNMASKED_LOOP;
        float sct[kNB];
#pragma unroll
        for (int t = 0; t < kNB; ++t) sct[t] = Kv::score_scale(qb[t], a.scale_log2);
        if constexpr (kSub == 1) {
          const typename Kv::Buf one[1] = {cur};
          consume_tiles<Kv, kCausal, kNB, 1, kMask>(st, one, qb, tok, t_end, sct, grp, lim);
        } else {
          consume_tiles<Kv, kCausal, kNB, kSub, kMask>(st, cur.s, qb, tok, t_end, sct, grp,
                                                       lim);
        }
      }
    };
    auto step_on = [&](const SBuf& cur, SBuf& nxt) {
      issue_span(nxt, g, tok + step, t_end, page_of(a, pt, r, tok + step, t_end));
#pragma unroll
      for (int t = 0; t < kNB; ++t) Kv::after_loads(qb[t]);
      compute(cur, std::false_type{});
      tok += step;
    };
    if (ns > 0) {
      for (int i = (ns - 1) >> 1; i > 0; --i) {
        step_on(buf[0], buf[1]);
        step_on(buf[1], buf[0]);
      }
      if ((ns & 1) == 0) {
        step_on(buf[0], buf[1]);
        buf[0] = buf[1];
      }
      compute(buf[0], std::true_type{});
    }
    // the next descriptor's query and first slice, the query first: as the
    // older load it is complete whenever the slice's first K row is, so the
    // next descriptor's loop can wait for its loads one by one
    if (has_next) {
#pragma unroll
      for (int t = 0; t < kNB; ++t) Kv::load_q(qb[t], a, ql[t], dn.x, dn.y, grp);
      issue_span(buf[0], dn.x, next_tok, dn.w, next_page);
    }

    // merge the wave states of this descriptor
#pragma unroll
    for (int t = 0; t < kNB; ++t) {
      const WaveState& w = st[t];
      const float l = wave_sum_across_groups(w.l);
      if (n < tile_cols(t)) {
        const int c = 16 * t + n;   // the column within this wave's columns
        if (grp == 0) {
          red[c] = w.m;
          red[16 * kNB + c] = l;
        }
        float* orow = red + kRedHead + c * kRedRow + 32 * grp;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          *reinterpret_cast<f32x4_t*>(orow + 8 * j) =
              f32x4_t{w.acc[0][j], w.acc[1][j], w.acc[2][j], w.acc[3][j]};
          *reinterpret_cast<f32x4_t*>(orow + 8 * j + 4) =
              f32x4_t{w.acc[4][j], w.acc[5][j], w.acc[6][j], w.acc[7][j]};
        }
      }
    }
    __syncthreads();
    // each thread merges four consecutive dims of one column (one float4 of
    // every wave's row), so an 8-column descriptor takes one pass of 256
    // threads; per dim the arithmetic is the same as one dim at a time
    constexpr int kD4 = kHeadDim / 4;
    for (int idx = threadIdx.x; idx < C * kD4; idx += kThreads) {
      const int q = idx / kD4, d4 = idx % kD4;
      // every wave's state of column q, all loads issued before the first
      // use (one LDS round trip instead of one per wave)
      float mw[kWaves], lw[kWaves];
      f32x4_t ow[kWaves];
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float* rw = smem + w * red_stride;
        mw[w] = rw[q];
        lw[w] = rw[16 * kNB + q];
        ow[w] = *reinterpret_cast<const f32x4_t*>(rw + kRedHead + q * kRedRow + 4 * d4);
      }
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mw[w]);
      // a column with no visible token in this descriptor (possible only
      // under a causal limit) gives an empty partial: o = 0, lse = -inf
      const float Mu = kCausal ? finite_or_zero(M) : M;
      float L = 0.f;
      f32x4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float c = __builtin_amdgcn_exp2f(mw[w] - Mu);
        L += lw[w] * c;
        o += ow[w] * c;
      }
      const bool empty = kCausal && !(L > 0.f);
      // one division for the four dims (each then one rounding more than a
      // division per dim: far inside the partials' float tolerance)
      const f32x4_t on = empty ? f32x4_t{0.f, 0.f, 0.f, 0.f} : o * (1.f / L);
      if (single) {
        // the pair's only descriptor: this is already the final output
        const int64_t row = kCausal ? query_row(r, g, q, a.q_len, G, a.num_q_heads)
                                    : int64_t(r) * a.num_q_heads + int64_t(g) * G + q;
        store_bf16x4(a.out, row, d4, on);
      } else {
        float* po = a.o_part + (int64_t(d) * C + q) * kHeadDim + 4 * d4;
        float* pl = a.lse_part + int64_t(d) * C + q;
        const float lse = empty ? -INFINITY : M + __builtin_amdgcn_logf(L);
        if constexpr (kFuse) {
          // merged inside this launch, possibly by a workgroup on another XCD
          const SplitRsrc sr = split_rsrc(a);
          store_row_coherent(sr, int64_t(d) * C + q, d4, on);
          if (d4 == 0) store_lse_coherent(sr, int64_t(d) * C + q, lse);
        } else {
          *reinterpret_cast<f32x4_t*>(po) = on;
          if (d4 == 0) *pl = lse;
        }
      }
    }
    __syncthreads();
    ds = dn;
  }
}

// ---------------------------------------------------------------------------
// merge of split pairs inside the kernel
// ---------------------------------------------------------------------------

constexpr int kFanIn = 16;        // partials one workgroup merges per query row and level
constexpr int kMergeUnroll = 8;   // partial rows in flight per thread

// Group size of the merge tree of a pair with cnt >= 2 partials: one group of
// all of them up to kFanIn, else the smallest f >= kFanIn with f*f >= cnt.
__device__ inline int merge_group_size(int cnt) {
  if (cnt <= kFanIn) return cnt;
  int f = kFanIn;
  while (f * f < cnt) ++f;
  return f;
}

// LDS floats the merge needs: per (row group, head) a max, a sum and a row.
constexpr int merge_lds_floats(int threads) { return 64 + (threads / 32) * kHeadDim; }

// Merges, for chunk columns q0 .. q0 + Cc - 1, the n partials in slots
// slot0, slot0 + stride, ... (in that order) of pair (g, r).  dst < 0: the
// result is the pair's final output (BF16 to `out`); otherwise it is written
// back as a partial (row and log-sum-exp) to slot dst.  Thread t owns float4
// column t % 32 of column q0 + (t / 32) % Cc and partials i = row group
// (mod R), R = threads / (32 Cc); the R states are merged through LDS in a
// fixed order, so the result is bitwise reproducible.
template <int kThreads>
__device__ void merge_columns(const AttendArgs& a, float* smem, int slot0, int stride, int n,
                              int dst, int g, int r, int q0, int Cc) {
  const int C = a.ncols;       // columns: query token q / G, head q % G
  const int R = kThreads / (32 * Cc);
  const int t = threadIdx.x;
  const int c4 = t & 31;
  const int qc = (t >> 5) % Cc;
  const int q = q0 + qc;
  const int rg = (t >> 5) / Cc;
  float m = -INFINITY, l = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  const SplitRsrc sr = split_rsrc(a);
  if (rg < R) {
    for (int i0 = rg; i0 < n; i0 += kMergeUnroll * R) {
      float ls[kMergeUnroll];
      f32x4_t v[kMergeUnroll];
#pragma unroll
      for (int u = 0; u < kMergeUnroll; ++u) {
        const int i = i0 + u * R;
        if (i < n) {
          const int64_t e = int64_t(slot0 + i * stride) * C + q;
          ls[u] = load_lse_coherent(sr, e);
          v[u] = load_row_coherent(sr, e, c4);
        }
      }
#pragma unroll
      for (int u = 0; u < kMergeUnroll; ++u)
        if (i0 + u * R < n) merge_into(m, l, acc, ls[u], v[u]);
    }
  }
  float* red_m = smem;         // [R * Cc] (R * Cc <= threads / 32 <= 32)
  float* red_l = smem + 32;
  f32x4_t* red_o = reinterpret_cast<f32x4_t*>(smem + 64);   // [R * Cc][32]
  if (rg < R) {
    const int s = rg * Cc + qc;
    if (c4 == 0) {
      red_m[s] = m;
      red_l[s] = l;
    }
    red_o[s * 32 + c4] = acc;
  }
  __syncthreads();
  if (rg == 0) {
    float M = -INFINITY;
    for (int k = 0; k < R; ++k) M = fmaxf(M, red_m[k * Cc + qc]);
    const float Mu = finite_or_zero(M);
    float L = 0.f;
    f32x4_t tot = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < R; ++k) {
      const float c = __builtin_amdgcn_exp2f(red_m[k * Cc + qc] - Mu);   // 0 for an empty state
      L += red_l[k * Cc + qc] * c;
      tot += red_o[(k * Cc + qc) * 32 + c4] * c;
    }
    const bool empty = !(L > 0.f);   // no visible token in any merged partial
    const f32x4_t o = empty ? f32x4_t{0.f, 0.f, 0.f, 0.f} : tot / L;
    if (dst < 0) {
      store_bf16x4(a.out, query_row(r, g, q, a.q_len, a.group, a.num_q_heads), c4, o);
    } else {
      const int64_t e = int64_t(dst) * C + q;
      store_row_coherent(sr, e, c4, o);
      if (c4 == 0) store_lse_coherent(sr, e, empty ? -INFINITY : M + __builtin_amdgcn_logf(L));
    }
  }
  __syncthreads();
}

// Merges the n partials in slots slot0, slot0 + stride, ... of pair (g, r)
// for every query column, in chunks of at most threads / 32 columns (see
// merge_columns for dst).
template <int kThreads>
__device__ void merge_run(const AttendArgs& a, float* smem, int slot0, int stride, int n, int dst,
                          int g, int r) {
  constexpr int kSlots = kThreads / 32;
  const int C = a.ncols;
  for (int q0 = 0; q0 < C; q0 += kSlots)
    merge_columns<kThreads>(a, smem, slot0, stride, n, dst, g, r, q0, min(kSlots, C - q0));
}

// Waits until every device-coherent store of the workgroup has completed
// (each wave waits for its own vector memory operations, then all meet at
// the barrier), so they are visible on every XCD.
__device__ inline void publish_workgroup() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
}

// One arrival on `counter` (after publish_workgroup).  True, in every thread,
// for the workgroup whose arrival completes `target`; that workgroup resets
// the counter for the next launch.  Its later coherent loads are issued
// after the count has returned, so they see every arrived partial.
__device__ inline bool arrive(int32_t* counter, int target, int* flag) {
  if (threadIdx.x == 0) {
    const int old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == target - 1;
    if (last) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = last;
  }
  __syncthreads();
  return *flag != 0;
}

// After a bin is drained: arrivals (and, for the last arriver, the merge)
// for every split pair among its descriptors.  A dynamic bin is one run of
// flat tiles, so only its first and its last descriptor can belong to a pair
// split over several bins; both are published together (one wait for the
// workgroup's stores) and their arrivals are counted in parallel, by two
// waves, so that a bin with two split pairs pays one chain, not two.
template <int kThreads>
__device__ void finish_split_pairs(const AttendArgs& a, const int4* __restrict__ descs,
                                   const int32_t* __restrict__ pair_count,
                                   const int32_t* __restrict__ pair_first, float* smem, int* flag,
                                   int d_begin, int d_end) {
  int sd[2];
  int nsd = 0;
  for (int d = d_begin; d < d_end; d = (d == d_begin && d_end - 1 > d_begin) ? d_end - 1 : d_end) {
    const int4 ds = descs[d];
    if (pair_count[ds.x * a.batch + ds.y] >= 2) sd[nsd++] = d;
  }
  if (nsd == 0) return;
  publish_workgroup();
  // the first arrival of each split descriptor: at its group's counter when
  // the pair merges in two levels, else at the pair's
  for (int j = 0; j < nsd; ++j) {
    if (int(threadIdx.x) != 64 * j) continue;
    const int4 ds = descs[sd[j]];
    const int p = ds.x * a.batch + ds.y;
    const int cnt = pair_count[p];
    const int first = pair_first[p];
    const int f = merge_group_size(cnt);
    int32_t* counter;
    int target;
    if ((cnt + f - 1) / f > 1) {
      const int lead = first + (sd[j] - first) / f * f;
      counter = a.arrive_group + lead;
      target = min(f, first + cnt - lead);
    } else {
      counter = a.arrive_pair + first;
      target = cnt;
    }
    const int old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == target - 1;
    if (last) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    flag[1 + j] = last;
  }
  __syncthreads();
  const bool last0 = flag[1] != 0, last1 = nsd > 1 && flag[2] != 0;
  __syncthreads();   // the flags are read before any later arrival rewrites them
  for (int j = 0; j < nsd; ++j) {
    if (!(j == 0 ? last0 : last1)) continue;
    const int4 ds = descs[sd[j]];
    const int p = ds.x * a.batch + ds.y;
    const int cnt = pair_count[p];
    const int first = pair_first[p];
    const int f = merge_group_size(cnt);
    const int ngroups = (cnt + f - 1) / f;
    if (ngroups == 1) {
      merge_run<kThreads>(a, smem, first, 1, cnt, -1, ds.x, ds.y);
      continue;
    }
    // level 1: this descriptor's group, into the group's first slot; level 2
    // (for the last group to finish): the group results, into `out`
    const int lead = first + (sd[j] - first) / f * f;
    merge_run<kThreads>(a, smem, lead, 1, min(f, first + cnt - lead), lead, ds.x, ds.y);
    publish_workgroup();
    if (arrive(a.arrive_pair + first, ngroups, flag))
      merge_run<kThreads>(a, smem, first, f, ngroups, -1, ds.x, ds.y);
  }
}

// One workgroup per persistent slot.  With grab_counter == null workgroup b
// drains bin b (the launch has one workgroup per bin).  Otherwise the launch
// has fewer workgroups than bins and each takes the next bin in increasing
// order from an atomic ticket counter until the bins run out, so a workgroup
// on a faster CU simply drains more bins; every workgroup draws exactly one
// ticket past the last bin, and the one holding the final ticket returns the
// counter to zero for the next launch.
// The decode instance (no causal limit, one column tile, merge in a second
// launch) carries drain_waves for bins of many short descriptors.  Its code
// costs short launches that never use it 0.1-0.4 us; a bin that needs it
// saves about a microsecond per descriptor past the first few.
// kFuse: the instance of the single-launch form, which merges split pairs
// itself (finish_split_pairs); the other instances leave the merge to the
// combine kernel and carry none of its code (about 2400 of the decode
// kernel's 4100 instructions, which measurably lengthen every launch
// although they never run there).
// One workgroup runs per CU (persistent bins), so more waves per SIMD than
// its own (waves / 4, rounded up) can never be resident.  Saying so pins the
// compiler's occupancy target: otherwise its scheduler squeezes the slice
// loop's registers toward occupancies that never occur, and whenever that
// loop is the kernel's register peak it stops issuing the next slice ahead
// of the current slice's math.
template <class Kv, bool kCausal, int kNB, int kTileW, bool kFuse>
__global__ __launch_bounds__((waves_of<Kv, kTileW>() * 64))
__attribute__((amdgpu_waves_per_eu((waves_of<Kv, kTileW>() + 3) / 4,
                                   (waves_of<Kv, kTileW>() + 3) / 4))) void attend_kernel(
    AttendArgs a, const int32_t* __restrict__ page_table, const int4* __restrict__ descs,
    const int32_t* __restrict__ pair_count, const int32_t* __restrict__ bin_offset,
    const int32_t* __restrict__ pair_first, const int4* __restrict__ bin_first) {
  constexpr int kThreads = waves_of<Kv, kTileW>() * 64;
  extern __shared__ __attribute__((aligned(16))) float smem[];   // f32x4 rows are stored in it
  __shared__ int ticket_lds;
  __shared__ int arrive_lds[3];   // the merge's arrival flags
  uint64_t t_start = 0;
  if (a.trace) t_start = __builtin_amdgcn_s_memrealtime();
  int drained = 0;
  // the first bin: this workgroup's own, or the first ticket
  auto next_bin = [&]() {
    if (threadIdx.x == 0) ticket_lds = atomicAdd(a.grab_counter, 1);
    __syncthreads();
    const int ticket = ticket_lds;
    __syncthreads();
    if (ticket >= a.num_bins && threadIdx.x == 0 && ticket == a.num_bins + int(gridDim.x) - 1)
      atomicExch(a.grab_counter, 0);
    return ticket;
  };
  int bin = a.grab_counter ? next_bin() : int(blockIdx.x);
  while (bin < a.num_bins) {
    attend_bin<Kv, kCausal, kNB, kTileW, kFuse>(a, page_table, descs, pair_count, bin_offset,
                                                bin_first, pair_first, smem, bin);
    const int d_begin = bin_offset[bin], d_end = bin_offset[bin + 1];
    if constexpr (kFuse)
      finish_split_pairs<kThreads>(a, descs, pair_count, pair_first, smem, arrive_lds, d_begin,
                                   d_end);
    drained += d_end - d_begin;
    if (!a.grab_counter) break;
    bin = next_bin();
  }

  // pairs without tokens: zero output rows (strided over the workgroups)
  const int npairs = a.num_kv_heads * a.batch;
  for (int p = blockIdx.x; p < npairs; p += gridDim.x) {
    if (pair_count[p] != 0) continue;
    const int g = p / a.batch, r = p % a.batch;
    for (int j = 0; j < a.q_len; ++j) {   // the group's rows of every query token
      uint4* rows = reinterpret_cast<uint4*>(
          static_cast<char*>(a.out) +
          query_row(r, g, j * a.group, a.q_len, a.group, a.num_q_heads) * kHeadDim * 2);
      for (int i = threadIdx.x; i < a.group * kHeadDim * 2 / 16; i += kThreads)
        rows[i] = make_uint4(0, 0, 0, 0);
    }
  }

  if (a.trace && threadIdx.x == 0) {
    uint32_t hw, xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    const uint64_t t_end = __builtin_amdgcn_s_memrealtime();
    uint64_t* t = a.trace + 4 * int64_t(blockIdx.x);
    t[0] = t_start;
    t[1] = t_end;
    t[2] = (uint64_t(xcc) << 32) | hw;
    t[3] = uint64_t(drained);
  }
}

}  // namespace

// The instance for a KV format: decode, or causal with 1-4 MFMA column
// tiles per wave (q_len > 1: at most 16, 32, 48 or 64 columns), with or
// without the in-kernel merge; its wave count.
template <class Kv, bool kFuse>
void pick_instance(bool causal, int tiles, const void** fn, int* waves) {
  *waves = Kv::kWaves;
  if (tiles == 4) {
    *fn = reinterpret_cast<const void*>(&attend_kernel<Kv, true, 4, kTileWaves, kFuse>);
    *waves = waves_of<Kv, kTileWaves>();
  } else if (tiles == 3) {
    *fn = reinterpret_cast<const void*>(&attend_kernel<Kv, true, 3, kTileWaves, kFuse>);
    *waves = waves_of<Kv, kTileWaves>();
  } else if (tiles == 2) {
    *fn = reinterpret_cast<const void*>(&attend_kernel<Kv, true, 2, Kv::kTile2Waves, kFuse>);
    *waves = waves_of<Kv, Kv::kTile2Waves>();
  } else {
    *fn = causal ? reinterpret_cast<const void*>(&attend_kernel<Kv, true, 1, 0, kFuse>)
                 : reinterpret_cast<const void*>(&attend_kernel<Kv, false, 1, 0, kFuse>);
  }
}
template <class Kv>
void pick_instance(bool causal, int tiles, bool fuse, const void** fn, int* waves) {
  if (fuse)
    pick_instance<Kv, true>(causal, tiles, fn, waves);
  else
    pick_instance<Kv, false>(causal, tiles, fn, waves);
}

hipError_t launch_attend(const AttendArgs& a, AttendKind kind, int grid, hipStream_t s) {
  AttendArgs copy = a;
  const int32_t* pt = a.page_table;
  const int4* descs = reinterpret_cast<const int4*>(a.desc);
  const int32_t* pc = a.pair_count;
  const int32_t* bo = a.bin_offset;
  const int32_t* pf = a.pair_first;
  const int4* bf = reinterpret_cast<const int4*>(a.bin_first);
  void* args[] = {&copy, &pt, &descs, &pc, &bo, &pf, &bf};
  // multi-token verification (q_len > 1) runs the instances with the causal
  // limit, one MFMA column tile per wave per 16 query columns; plain decode
  // keeps the loop without it
  const bool causal = a.q_len > 1;
  if (a.ncols < 1 || a.ncols > 64 || (!causal && a.ncols > 16)) return hipErrorInvalidValue;
  const int tiles = causal ? (a.ncols + 15) / 16 : 1;
  int waves;
  const void* fn;
  switch (kind) {
    case kAttendFp8:
      pick_instance<Fp8Kv>(causal, tiles, a.fuse != 0, &fn, &waves);
      break;
    case kAttendFp8Q8:
      pick_instance<Fp8KvQ8>(causal, tiles, a.fuse != 0, &fn, &waves);
      break;
    default:
      pick_instance<Bf16Kv>(causal, tiles, a.fuse != 0, &fn, &waves);
  }
  // per wave for the merge: m and l of 16 tiles columns, then the C rows
  size_t lds = size_t(waves) * (32 * tiles + size_t(a.ncols) * kRedRow) * sizeof(float);
  const size_t merge_lds = size_t(merge_lds_floats(waves * 64)) * sizeof(float);
  if (a.fuse && merge_lds > lds) lds = merge_lds;
  if (grid <= 0) return hipSuccess;
  return hipLaunchKernel(fn, dim3(grid), dim3(waves * 64), args, lds, s);
}

}  // namespace lbp
