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

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  __shared__ int scan_lds[kPlanWaves];
  __shared__ int flag_lds;
  const int tid = threadIdx.x;
  const int B = a.batch;
  const int npairs = a.num_kv_heads * B;
  const int chunk = (npairs + kPlanThreads - 1) / kPlanThreads;
  const int p0 = min(tid * chunk, npairs);
  const int p1 = min(p0 + chunk, npairs);
  if (tid == 0) flag_lds = 0;

  // pass 1: tiles per pair, flat starts, total T
  int flag = 0;
  int local = 0;
  for (int p = p0; p < p1; ++p) {
    int L = clamp_len(a.seq_lens[p % B], a.max_tokens, &flag);
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
  int cnt_local = 0;
  for (int p = p0; p < p1; ++p) {
    int L = clamp_len(a.seq_lens[p % B], a.max_tokens, &flag);
    int n = (L + kPageTokens - 1) / kPageTokens;
    int cnt;
    if (dynamic) {
      cnt = n ? (start + n - 1) / budget - start / budget + 1 : 0;
      a.scratch[p] = start;
    } else if (a.policy == LBP_POLICY_STATIC_SPLITS) {
      int c = (n + budget - 1) / budget;          // ceil(n / S) tiles per split
      cnt = c ? (n + c - 1) / c : 0;
    } else {
      cnt = (n + budget - 1) / budget;            // ceil(n / C) chunks
    }
    a.pair_count[p] = cnt;
    cnt_local += cnt;
    start += n;
  }
  int D;
  int first = block_exclusive_scan(cnt_local, scan_lds, &D);
  for (int p = p0; p < p1; ++p) {
    a.pair_first[p] = first;
    first += a.pair_count[p];
  }
  // pairs split over several descriptors, compacted in pair order
  int nsplit_local = 0;
  for (int p = p0; p < p1; ++p) nsplit_local += a.pair_count[p] >= 2;
  int nsplit;
  int sfirst = block_exclusive_scan(nsplit_local, scan_lds, &nsplit);
  for (int p = p0; p < p1; ++p) {
    const int cnt = a.pair_count[p];
    if (cnt >= 2 && sfirst < a.max_split)
      reinterpret_cast<int4*>(a.split_list)[sfirst++] = make_int4(p, a.pair_first[p], cnt, 0);
  }
  __syncthreads();  // scratch / pair_first / pair_count visible to the block

  // arrival counters of the attention kernel's merge start at zero
  for (int i = tid; i < a.arrive_words; i += kPlanThreads) a.arrive[i] = 0;

  // descriptors, in parallel over descriptor slots
  for (int d = tid; d < D; d += kPlanThreads) {
    int p = last_le(a.pair_first, npairs, d);
    int j = d - a.pair_first[p];
    int r = p % B;
    int dummy = 0;
    int L = clamp_len(a.seq_lens[r], a.max_tokens, &dummy);
    int n = (L + kPageTokens - 1) / kPageTokens;
    int lo, hi;
    if (dynamic) {
      int S = a.scratch[p];
      int64_t bin = S / budget + j;
      lo = int(max<int64_t>(S, bin * budget) - S);
      hi = int(min<int64_t>(S + n, (bin + 1) * budget) - S);
    } else if (a.policy == LBP_POLICY_STATIC_SPLITS) {
      int c = (n + budget - 1) / budget;
      lo = j * c;
      hi = min(lo + c, n);
    } else {
      lo = j * budget;
      hi = min(lo + budget, n);
    }
    int4 v = make_int4(p / B, r, lo * kPageTokens, min(hi * kPageTokens, L));
    reinterpret_cast<int4*>(a.desc)[d] = v;
  }

  // per-bin descriptor offsets
  int U;
  if (dynamic) {
    U = T ? (T + budget - 1) / budget : 0;
    for (int b = tid; b <= a.num_bins; b += kPlanThreads) {
      int off;
      if (b >= U) {
        off = D;
      } else {
        int f = b * budget;          // < T, so fits in int
        int p = last_le(a.scratch, npairs, f);
        off = a.pair_first[p] + (b - a.scratch[p] / budget);
      }
      a.bin_offset[b] = off;
    }
  } else {
    U = D;
    const int S = a.splits_per_pair;
    for (int b = tid; b <= a.num_bins; b += kPlanThreads) {
      int off;
      if (b == a.num_bins) {
        off = D;
      } else {
        int p = b / S, s = b % S;
        off = a.pair_first[p] + min(s, a.pair_count[p]);
      }
      a.bin_offset[b] = off;
    }
  }

  __syncthreads();  // descriptors and bin offsets visible to the block
  // each bin's first descriptor, read by the attention kernel with its range
  for (int b = tid; b < a.num_bins; b += kPlanThreads) {
    const int d = a.bin_offset[b];
    int4 v = make_int4(0, 0, 0, 0);
    if (d < a.bin_offset[b + 1]) v = reinterpret_cast<const int4*>(a.desc)[d];
    reinterpret_cast<int4*>(a.bin_first)[b] = v;
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
  return hipLaunchKernel(reinterpret_cast<const void*>(&plan_kernel), dim3(1),
                         dim3(kPlanThreads), args, 0, s);
}

}  // namespace lbp
