// Task-map builders: the dynamic assign kernel and the static split-KV plans.
//
// Dynamic assign (SGLang x HPC-Ops page, "Scheduling around live KV work";
// vLLM x HPC-Ops page, "Solution: per-step load-balanced decode scheduler",
// bullet "Assign"): every (KV head, request) pair is cut into ceil(L/64)
// tiles; with T the total over all pairs and W the persistent workgroups,
// budget = max(ceil(T/W), F); pairs are laid end to end head-major,
// batch-minor, and flat tile f belongs to bin f / budget, so each bin fills
// to the budget before the next starts.  A descriptor is one run of one pair
// inside one bin.
//
// One workgroup of 1024 threads builds the whole map with integer arithmetic
// only, so the map is bit-identical to the greedy fill: the flat start S_p of
// each pair comes from a block-wide prefix sum, a pair touches bins
// S_p/budget .. (S_p+n_p-1)/budget (one descriptor each), descriptor slots
// come from a second prefix sum, and both the descriptors and the per-bin
// offsets are then produced in parallel by binary search.
#include "lbp_internal.h"

namespace lbp {
namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;

// Exclusive prefix sum over the block; *total receives the sum of all v.
__device__ int block_exclusive_scan(int v, int* lds, int* total) {
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) lds[wid] = x;
  __syncthreads();
  if (wid == 0) {
    int w = lane < kPlanWaves ? lds[lane] : 0;
#pragma unroll
    for (int off = 1; off < kPlanWaves; off <<= 1) {
      int y = __shfl_up(w, off, 64);
      if (lane >= off) w += y;
    }
    if (lane < kPlanWaves) lds[lane] = w;
  }
  __syncthreads();
  const int before = wid ? lds[wid - 1] : 0;
  *total = lds[kPlanWaves - 1];
  __syncthreads();
  return before + x - v;
}

__device__ inline int clamp_len(int L, int max_tokens, int* flag) {
  if (L < 0) return 0;
  if (L > max_tokens) { *flag = 1; return max_tokens; }
  return L;
}

// Index of the last element of a[0..n) (nondecreasing) that is <= key.
__device__ inline int last_le(const int32_t* a, int n, int key) {
  int lo = 0, hi = n;  // answer in [lo, hi)
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (a[mid] <= key) lo = mid; else hi = mid;
  }
  return lo;
}

// Per-pair arrays the builder reads back (clamped length, flat start, first
// descriptor, descriptor count) live in LDS when the batch fits, so the two
// binary searches and the re-reads between phases are LDS accesses instead
// of dependent global round trips; larger batches use the plan workspace.
constexpr int kLdsPairs = 8192;   // 4 x 4 B x 8192 = 128 KB

template <bool kLds>
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  __shared__ int scan_lds[kPlanWaves];
  __shared__ int flag_lds;
  extern __shared__ int pair_lds[];   // kLds: len, start, first, count [npairs] each
  const int tid = threadIdx.x;
  const int B = a.batch;
  const int npairs = a.num_kv_heads * B;
  const int chunk = (npairs + kPlanThreads - 1) / kPlanThreads;
  const int p0 = min(tid * chunk, npairs);
  const int p1 = min(p0 + chunk, npairs);
  int* const s_len = pair_lds;
  int* const start_of = kLds ? pair_lds + npairs : a.scratch;
  int* const first_of = kLds ? pair_lds + 2 * npairs : a.pair_first;
  int* const count_of = kLds ? pair_lds + 3 * npairs : a.pair_count;
  auto len_of = [&](int p) {
    if constexpr (kLds) {
      return s_len[p];
    } else {
      int unused = 0;
      return clamp_len(a.seq_lens[p % B], a.max_tokens, &unused);
    }
  };
  if (tid == 0) flag_lds = 0;

  // pass 1: tiles per pair, flat starts, total T
  int flag = 0;
  int local = 0;
  for (int p = p0; p < p1; ++p) {
    const int L = clamp_len(a.seq_lens[p % B], a.max_tokens, &flag);
    if constexpr (kLds) s_len[p] = L;
    local += (L + kPageTokens - 1) / kPageTokens;
  }
  int T;
  int start = block_exclusive_scan(local, scan_lds, &T);
  if (flag) atomicOr(&flag_lds, 1);

  const bool dynamic = a.policy == LBP_POLICY_DYNAMIC;
  int budget;
  if (dynamic) {
    budget = max((T + a.num_bins - 1) / a.num_bins, a.param);
  } else {
    budget = a.param;
  }

  // pass 2: descriptors per pair
  int cnt_local = 0, nsplit_local = 0;
  for (int p = p0; p < p1; ++p) {
    const int n = (len_of(p) + kPageTokens - 1) / kPageTokens;
    int cnt;
    if (dynamic) {
      cnt = n ? (start + n - 1) / budget - start / budget + 1 : 0;
      start_of[p] = start;
    } else if (a.policy == LBP_POLICY_STATIC_SPLITS) {
      int c = (n + budget - 1) / budget;          // ceil(n / S) tiles per split
      cnt = c ? (n + c - 1) / c : 0;
    } else {
      cnt = (n + budget - 1) / budget;            // ceil(n / C) chunks
    }
    count_of[p] = cnt;
    if constexpr (kLds) a.pair_count[p] = cnt;
    cnt_local += cnt;
    nsplit_local += cnt >= 2;
    start += n;
  }
  int D;
  int first = block_exclusive_scan(cnt_local, scan_lds, &D);
  for (int p = p0; p < p1; ++p) {
    first_of[p] = first;
    if constexpr (kLds) a.pair_first[p] = first;
    first += count_of[p];
  }
  // pairs split over several descriptors, compacted in pair order
  int nsplit;
  int sfirst = block_exclusive_scan(nsplit_local, scan_lds, &nsplit);
  for (int p = p0; p < p1; ++p) {
    const int cnt = count_of[p];
    if (cnt >= 2 && sfirst < a.max_split)
      reinterpret_cast<int4*>(a.split_list)[sfirst++] = make_int4(p, first_of[p], cnt, 0);
  }
  __syncthreads();  // the per-pair arrays visible to the block

  // arrival counters of the attention kernel's merge start at zero
  for (int i = tid; i < a.arrive_words; i += kPlanThreads) a.arrive[i] = 0;

  // descriptor j of pair p
  auto desc_of = [&](int p, int j) {
    const int r = p % B;
    const int L = len_of(p);
    const int n = (L + kPageTokens - 1) / kPageTokens;
    int lo, hi;
    if (dynamic) {
      const int S = start_of[p];
      const int64_t bin = S / budget + j;
      lo = int(max<int64_t>(S, bin * budget) - S);
      hi = int(min<int64_t>(S + n, (bin + 1) * budget) - S);
    } else if (a.policy == LBP_POLICY_STATIC_SPLITS) {
      const int c = (n + budget - 1) / budget;
      lo = j * c;
      hi = min(lo + c, n);
    } else {
      lo = j * budget;
      hi = min(lo + budget, n);
    }
    return make_int4(p / B, r, lo * kPageTokens, min(hi * kPageTokens, L));
  };

  // descriptors, in parallel over descriptor slots
  for (int d = tid; d < D; d += kPlanThreads) {
    const int p = last_le(first_of, npairs, d);
    reinterpret_cast<int4*>(a.desc)[d] = desc_of(p, d - first_of[p]);
  }

  // per-bin descriptor offsets, and each bin's first descriptor (read by
  // the attention kernel together with the range), computed in place
  int U;
  int4* const bin_first = reinterpret_cast<int4*>(a.bin_first);
  if (dynamic) {
    U = T ? (T + budget - 1) / budget : 0;
    for (int b = tid; b <= a.num_bins; b += kPlanThreads) {
      int off = D;
      int4 v = make_int4(0, 0, 0, 0);
      if (b < U) {                   // a used bin holds at least one descriptor
        const int f = b * budget;    // < T, so fits in int
        const int p = last_le(start_of, npairs, f);
        const int j = b - start_of[p] / budget;
        off = first_of[p] + j;
        v = desc_of(p, j);
      }
      a.bin_offset[b] = off;
      if (b < a.num_bins) bin_first[b] = v;
    }
  } else {
    U = D;
    const int S = a.splits_per_pair;
    for (int b = tid; b <= a.num_bins; b += kPlanThreads) {
      int off = D;
      int4 v = make_int4(0, 0, 0, 0);
      if (b < a.num_bins) {
        const int p = b / S, s = b % S;
        off = first_of[p] + min(s, count_of[p]);
        if (s < count_of[p]) v = desc_of(p, s);
        bin_first[b] = v;
      }
      a.bin_offset[b] = off;
    }
  }

  if (tid == 0) {
    int32_t* h = a.header;
    h[kHdrMagic] = int32_t(LBP_PLAN_MAGIC);
    h[kHdrPolicy] = a.policy;
    h[kHdrNumBins] = a.num_bins;
    h[kHdrBatch] = B;
    h[kHdrKvHeads] = a.num_kv_heads;
    h[kHdrTiles] = T;
    h[kHdrBudget] = budget;
    h[kHdrDesc] = D;
    h[kHdrUsedBins] = U;
    h[kHdrStatus] = flag_lds ? kStatusClamped : 0;
    for (int i = kHdrStatus + 1; i < kHdrWords; ++i) h[i] = 0;
    h[kHdrSplits] = min(nsplit, a.max_split);
  }
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  PlanArgs copy = a;
  void* args[] = {&copy};
  const int npairs = a.num_kv_heads * a.batch;
  if (npairs <= kLdsPairs)
    return hipLaunchKernel(reinterpret_cast<const void*>(&plan_kernel<true>), dim3(1),
                           dim3(kPlanThreads), args, size_t(npairs) * 16, s);
  return hipLaunchKernel(reinterpret_cast<const void*>(&plan_kernel<false>), dim3(1),
                         dim3(kPlanThreads), args, 0, s);
}

}  // namespace lbp
