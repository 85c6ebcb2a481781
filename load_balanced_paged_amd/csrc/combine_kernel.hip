// LSE combine of split-KV partials into the final BF16 output.
//
// Method (SGLang x HPC-Ops page, "Scheduling around live KV work", second
// paragraph; vLLM x HPC-Ops page, bullet "Compute and combine"): for every
// (KV head, request) pair the combine reads how many partials the task map
// gave it and merges them under the global softmax normalisation:
// with M = max_k lse_k and w_k = 2^(lse_k - M),
// out = sum_k w_k o_k / sum_k w_k (base-2 log-sum-exp of log2(e)-scaled
// scores, as the attention kernel writes them), rounded to BF16 (nearest
// even).
//
// gfx950 mapping: only pairs that were really split need merging (a pair
// with one descriptor is finished in place by the attention kernel, a pair
// with none is zero-filled there too), and the plan lists them compactly:
// (pair, first descriptor, count).  A dynamic plan splits at most W - 1 pairs
// (one per internal bin boundary), so the grid is (min(pairs, W - 1), C)
// regardless of batch size, C = G * q_len query columns; workgroup (i, q)
// merges column q (query token q / G, head q % G) of list entry i, or exits
// if the plan has fewer entries.  Thread t owns dims
// [4(t%32), +4) of partials k = t/32 (mod R), R = threads / 32, and loads
// each partial's log-sum-exp together with its row, sixteen partials per
// thread in flight, and merges each round of loads at once (one rescale of
// the running max, sum and accumulator per round, one exp2 per partial):
// 16 R partial rows per round trip, so the critical path is the launch plus
// two dependent memory round trips (the list entry, then the rows) for up to
// 16 R splits.  The R per-thread states are merged in LDS in a fixed order
// (bitwise deterministic).  Workgroups have 256 threads (128 rows per round
// trip); a grid of at most one workgroup per CU, which few split pairs with
// many partials each give, uses 512 (256 rows): the wider workgroups cost
// dispatch time only when there are many of them.  When the list can hold
// more than 32 pairs of at least 8 columns, or more than 256 / C pairs of
// fewer (decode at G <= 8, or verification: many split pairs of few
// partials), combine_pairs_kernel runs instead, one workgroup per pair and
// chunk of 8 columns.
#include "lse_merge.h"

namespace lbp {
namespace {

constexpr int kLanesPerRow = kHeadDim / 4;              // 32 float4 per 128-dim row
constexpr int kUnroll = 16;
constexpr int kWideGrid = 256;   // workgroups up to which the 512-thread form runs

// Merges the first n of N loaded (lse, row) pairs into a running (max, sum,
// acc) state at once: the state is rescaled once to the round's new maximum,
// then every partial adds 2^(lse - max) times its row, one exp2 each instead
// of the two and the rescale of an online merge per partial.  Empty partials
// (lse = -inf) add nothing; an all-empty state stays (-inf, 0, 0).
template <int N>
__device__ inline void merge_round(float& m, float& l, f32x4_t& acc, const float (&ls)[N],
                                   const f32x4_t (&v)[N], int n) {
  float mr = m;
#pragma unroll
  for (int u = 0; u < N; ++u)
    if (u < n) mr = fmaxf(mr, ls[u]);
  const float ref = finite_or_zero(mr);
  const float a = __builtin_amdgcn_exp2f(m - ref);   // 0 while the state is empty
  acc = acc * a;
  l = l * a;
#pragma unroll
  for (int u = 0; u < N; ++u) {
    if (u < n) {
      const float b = __builtin_amdgcn_exp2f(ls[u] - ref);
      acc += v[u] * b;
      l += b;
    }
  }
  m = mr;
}

template <int kThreads>
__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  constexpr int kRowGroups = kThreads / kLanesPerRow;     // partial rows per sweep
  __shared__ float red_m[kRowGroups];
  __shared__ float red_l[kRowGroups];
  __shared__ f32x4_t red_o[kRowGroups][kLanesPerRow];

  // The grid never exceeds the list's capacity, so the entry can be loaded
  // together with the entry count (one round trip instead of two).
  const int nsplit = a.header[kHdrSplits];
  const int4 e = reinterpret_cast<const int4*>(a.split_list)[blockIdx.x];
  asm volatile("" ::"s"(e.x), "s"(e.y), "s"(e.z));   // keeps the entry load above the exit
  if (int(blockIdx.x) >= nsplit) return;
  const int p = e.x;             // pair = kv_head * batch + request
  const int first = e.y;
  const int cnt = e.z;           // >= 2
  const int q = blockIdx.y;      // column: query token q / G, head q % G of the group
  const int C = a.ncols;
  const int g = p / a.batch, r = p % a.batch;
  const int64_t row = query_row(r, g, q, a.q_len, a.group, a.num_q_heads);
  const int t = threadIdx.x;
  const int c4 = t % kLanesPerRow;
  const int kg = t / kLanesPerRow;
  const float* lse = a.lse_part + int64_t(first) * C + q;
  const f32x4_t* o = reinterpret_cast<const f32x4_t*>(a.o_part + (int64_t(first) * C + q) * kHeadDim);
  const int64_t stride4 = int64_t(C) * kLanesPerRow;   // float4s between consecutive partials

  float m = -INFINITY, l = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = kg; k0 < cnt; k0 += kUnroll * kRowGroups) {
    float ls[kUnroll];
    f32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int k = k0 + u * kRowGroups;
      if (k < cnt) {
        ls[u] = lse[int64_t(k) * C];
        v[u] = o[int64_t(k) * stride4 + c4];
      }
    }
    merge_round(m, l, acc, ls, v, (cnt - k0 + kRowGroups - 1) / kRowGroups);
  }
  if (c4 == 0) {
    red_m[kg] = m;
    red_l[kg] = l;
  }
  red_o[kg][c4] = acc;
  __syncthreads();
  if (kg != 0) return;
  float M = -INFINITY;
#pragma unroll
  for (int i = 0; i < kRowGroups; ++i) M = fmaxf(M, red_m[i]);
  const float Mu = finite_or_zero(M);
  float L = 0.f;
  f32x4_t tot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < kRowGroups; ++i) {
    const float c = __builtin_amdgcn_exp2f(red_m[i] - Mu);   // 0 for threads that saw no partial
    L += red_l[i] * c;
    tot += red_o[i][c4] * c;
  }
  // a query token with no visible KV position (causal verification) outputs 0
  store_bf16x4(a.out, row, c4, L > 0.f ? tot / L : f32x4_t{0.f, 0.f, 0.f, 0.f});
}

// One workgroup per split pair and chunk of 8 query columns, for many pairs
// of few partials each: 32 threads per column (one float4 of the row each),
// each merging its column's partials in order, kPairUnroll in flight.  One
// workgroup per 8 columns instead of one per column makes the grid 8 times
// smaller.
constexpr int kPairThreads = 256;
constexpr int kPairUnroll = 8;
constexpr int kPairCols = kPairThreads / kLanesPerRow;   // 8

__global__ __launch_bounds__(kPairThreads) void combine_pairs_kernel(CombineArgs a) {
  const int nsplit = a.header[kHdrSplits];
  const int4 e = reinterpret_cast<const int4*>(a.split_list)[blockIdx.x];
  asm volatile("" ::"s"(e.x), "s"(e.y), "s"(e.z));   // keeps the entry load above the exit
  if (int(blockIdx.x) >= nsplit) return;
  const int p = e.x, first = e.y, cnt = e.z;
  const int C = a.ncols;
  const int q = int(blockIdx.y) * kPairCols + int(threadIdx.x) / kLanesPerRow;
  const int c4 = threadIdx.x % kLanesPerRow;
  if (q >= C) return;
  const int g = p / a.batch, r = p % a.batch;
  const float* lse = a.lse_part + int64_t(first) * C + q;
  const f32x4_t* o = reinterpret_cast<const f32x4_t*>(a.o_part + (int64_t(first) * C + q) * kHeadDim);
  const int64_t stride4 = int64_t(C) * kLanesPerRow;
  float m = -INFINITY, l = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < cnt; k0 += kPairUnroll) {
    float ls[kPairUnroll];
    f32x4_t v[kPairUnroll];
#pragma unroll
    for (int u = 0; u < kPairUnroll; ++u) {
      if (k0 + u < cnt) {
        ls[u] = lse[int64_t(k0 + u) * C];
        v[u] = o[int64_t(k0 + u) * stride4 + c4];
      }
    }
    merge_round(m, l, acc, ls, v, cnt - k0);
  }
  store_bf16x4(a.out, query_row(r, g, q, a.q_len, a.group, a.num_q_heads), c4,
               l > 0.f ? acc / l : f32x4_t{0.f, 0.f, 0.f, 0.f});
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, int max_split, hipStream_t s) {
  if (max_split <= 0) return hipSuccess;
  CombineArgs copy = a;
  void* args[] = {&copy};
  // many possible split pairs: few partials each (the plan splits at most
  // W - 1 times in all), so one workgroup per pair and 8 columns
  if (int64_t(max_split) * (a.ncols < kPairCols ? a.ncols : kPairCols) > kWideGrid)
    return hipLaunchKernel(reinterpret_cast<const void*>(&combine_pairs_kernel),
                           dim3(max_split, (a.ncols + kPairCols - 1) / kPairCols),
                           dim3(kPairThreads), args, 0, s);
  const bool wide = int64_t(max_split) * a.ncols <= kWideGrid;
  const void* fn = wide ? reinterpret_cast<const void*>(&combine_kernel<512>)
                        : reinterpret_cast<const void*>(&combine_kernel<256>);
  return hipLaunchKernel(fn, dim3(max_split, a.ncols), dim3(wide ? 512 : 256), args, 0, s);
}

}  // namespace lbp
