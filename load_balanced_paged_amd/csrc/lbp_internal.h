// Internal definitions shared by the host API and the HIP kernels of liblbp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lbp.h"

namespace lbp {

constexpr int kHeadDim = LBP_HEAD_DIM;   // 128
constexpr int kPageTokens = LBP_PAGE_SIZE;  // 64: one page is one scheduling tile
constexpr int kMaxGroup = LBP_MAX_GROUP;    // query heads per KV head, padded to 16 MFMA rows
// F, the minimum-work floor (tiles per bin) when the config leaves it 0: 1,
// no floor.  A small batch's attention is latency-bound here and the combine
// is one launch of at most W - 1 pairs whatever the split count, so fewer,
// larger bins measured slower (up to 1.5 us on a one-request batch).
constexpr int kDefaultMinTiles = 1;

// header word indices inside the plan workspace
enum HeaderWord {
  kHdrMagic = 0, kHdrPolicy = 1, kHdrNumBins = 2, kHdrBatch = 3, kHdrKvHeads = 4,
  kHdrTiles = 5, kHdrBudget = 6, kHdrDesc = 7, kHdrUsedBins = 8, kHdrStatus = 9,
  kHdrTicket = 10,  // bin ticket counter of the attention kernel (zero between launches)
  kHdrSplits = 11,  // number of entries in the split-pair list
  kHdrWords = 16
};
constexpr int kStatusClamped = 1;

inline uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

// Capacity of the split-pair list.  In a dynamic plan a pair is split only
// if one of the U - 1 <= W - 1 internal bin boundaries falls inside it, so at
// most W - 1 pairs are split; a static plan may split every pair.
inline int max_split_pairs(int policy, int num_bins, int npairs) {
  if (policy == LBP_POLICY_DYNAMIC) return npairs < num_bins - 1 ? npairs : num_bins - 1;
  return npairs;
}

// Arrival counters of the in-kernel merge of split pairs (dynamic plans):
// one per descriptor slot for the pair level and one for the group level.
inline int arrive_words(int policy, int max_desc) {
  return policy == LBP_POLICY_DYNAMIC ? 2 * max_desc : 0;
}

// Byte layout of the task map for one plan.
// The header words directly precede the bin offsets in every plan workspace
// (below), so a kernel holding bin_offset reads header word i at
// bin_offset[i - kHdrWords].
static_assert(kHdrWords * 4 % 64 == 0, "the bin offsets follow the header directly");
inline lbp_plan_offsets plan_layout(int policy, int num_bins, int max_desc, int npairs) {
  lbp_plan_offsets o;
  o.header = 0;
  o.bin_offset = align_up(o.header + kHdrWords * 4, 64);
  o.bin_first = align_up(o.bin_offset + uint64_t(num_bins + 1) * 4, 64);
  o.desc = align_up(o.bin_first + uint64_t(num_bins) * 32, 64);
  o.pair_first = align_up(o.desc + uint64_t(max_desc) * 16, 64);
  o.pair_count = align_up(o.pair_first + uint64_t(npairs) * 4, 64);
  o.scratch = align_up(o.pair_count + uint64_t(npairs) * 4, 64);
  o.split_list = align_up(o.scratch + uint64_t(npairs) * 4, 64);
  o.arrive = align_up(o.split_list + uint64_t(max_split_pairs(policy, num_bins, npairs)) * 16, 64);
  o.total = align_up(o.arrive + uint64_t(arrive_words(policy, max_desc)) * 4, 256);
  return o;
}

// Split buffer: o_part[max_desc][C][128] fp32, then lse_part[max_desc][C]
// fp32, with C = G * q_len columns (query token c / G, head c % G).
inline uint64_t split_lse_offset(int max_desc, int ncols) {
  return align_up(uint64_t(max_desc) * ncols * kHeadDim * 4, 256);
}
inline uint64_t split_bytes(int max_desc, int ncols) {
  return align_up(split_lse_offset(max_desc, ncols) + uint64_t(max_desc) * ncols * 4, 256);
}

// Row of q / out ([B][q_len][Hq][128]) for column c of KV head g, request r.
__host__ __device__ inline int64_t query_row(int r, int g, int c, int q_len, int group,
                                             int num_q_heads) {
  return (int64_t(r) * q_len + c / group) * num_q_heads + int64_t(g) * group + c % group;
}

struct PlanArgs {
  const int32_t* seq_lens;
  int32_t batch, num_kv_heads, num_bins, policy, param;
  int32_t splits_per_pair;   // static policies: bins per pair
  int32_t max_tokens;        // 64 * max_pages_per_seq
  int32_t* header;
  int32_t* bin_offset;
  int32_t* bin_first;        // [num_bins][8]: each bin's first descriptor, then the pages
                             // of its first two tiles (the second clamped to the last), 0, 0
  const int32_t* page_table;
  int64_t page_table_stride;
  int32_t* desc;             // [max_desc][4]
  int32_t* pair_first;
  int32_t* pair_count;
  int32_t* scratch;          // first flat tile of every pair (dynamic)
  int32_t* split_list;       // [max_split][4]: (pair, first descriptor, count, 0)
  int32_t max_split;
  int32_t* arrive;           // arrival counters, zeroed here
  int32_t arrive_words;
};

struct AttendArgs {
  const int32_t* bin_offset;
  const int32_t* bin_first;
  const int32_t* desc;
  const int32_t* pair_count;
  const int32_t* pair_first;
  const int32_t* page_table;
  int64_t page_table_stride;
  const void* q;             // [B][Hq][128] bf16, or e4m3 codes with q_scale
  const float* q_scale;      // [B][Hq] fp32 scale of FP8 queries, else null
  const void* k_cache;       // [P][H_kv][64][128] bf16 or e4m3
  const void* v_cache;
  const float* k_scale;      // [P][H_kv][64] (FP8 only)
  const float* v_scale;
  float* o_part;             // [max_desc][G][128]
  float* lse_part;           // [max_desc][G]
  int32_t o_part_bytes;      // bytes of the two sections (the in-kernel merge
  int32_t lse_part_bytes;    // reads and writes them through buffer resources)
  void* out;                 // [B][Hq][128] bf16: single-descriptor pairs land here
  uint64_t* trace;           // optional [grid][4] workgroup records, or null
  int32_t* grab_counter;     // null: workgroup b drains bin b; else the ticket counter
  int32_t* arrive_pair;      // [max_desc] pair-level arrival counters (at pair_first)
  int32_t* arrive_group;     // [max_desc] group-level arrival counters (at the group's first slot)
  int32_t fuse;              // 1: merge split pairs in this kernel (dynamic plans)
  int32_t num_bins;
  int32_t batch, num_q_heads, num_kv_heads, group;
  int32_t q_len, ncols;      // query tokens per request; columns = group * q_len
  float scale_log2;          // sm_scale * log2(e)
};

struct CombineArgs {
  const int32_t* header;     // kHdrSplits = entries in split_list
  const int32_t* split_list;
  const float* o_part;
  const float* lse_part;
  void* out;                 // [B][q_len][Hq][128] bf16
  int32_t batch, num_q_heads, num_kv_heads, group;
  int32_t q_len, ncols;
};

struct PrologueArgs {
  const void* qkv;           // [B][(Hq + 2 Hkv) * 128] bf16
  const int32_t* seq_lens;
  const int32_t* page_table;
  int64_t page_table_stride;
  const float* q_norm_weight;
  const float* k_norm_weight;
  const float* rope_cos_sin; // [max_position][128]
  int32_t max_position;
  float norm_eps;
  int32_t q_fp8, kv_fp8;
  void* q_out;
  float* q_scale_out;
  void* k_cache;
  void* v_cache;
  float* k_scale;
  float* v_scale;
  int32_t batch, num_q_heads, num_kv_heads;
  int32_t q_len;             // new tokens per request
  int32_t max_tokens;        // 64 * max_pages_per_seq
};

// Launchers (defined next to their kernels).  Each returns the HIP error of
// the launch itself.
hipError_t launch_plan(const PlanArgs& a, hipStream_t s);
// Kernel instance: KV format and query precision.
enum AttendKind { kAttendBf16 = 0, kAttendFp8 = 1, kAttendFp8Q8 = 2 };
hipError_t launch_attend(const AttendArgs& a, AttendKind kind, int grid, hipStream_t s);
hipError_t launch_combine(const CombineArgs& a, int max_split, hipStream_t s);
hipError_t launch_prologue(const PrologueArgs& a, hipStream_t s);
hipError_t launch_read_stream(const void* src, int64_t n16, int32_t* sink, int blocks,
                              hipStream_t s);

}  // namespace lbp
