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
// only, so the map is bit-identical to the greedy fill.  A first sweep sums
// the tiles (T, hence the budget).  The pairs are then taken in rounds of
// 1024, one per thread, in pair order: a block-wide prefix sum over the
// round (plus the total of the rounds before) gives each pair's flat start
// S_p, and a second one over descriptor counts (a pair touches bins
// S_p/budget .. (S_p+n_p-1)/budget, one descriptor each) gives its first
// descriptor slot, so every per-pair load and store is coalesced.  A pair's
// first descriptor is written in its round.  Every other descriptor starts
// at a bin boundary inside a pair, and there are at most W - 1 of them, so
// those are written bin by bin: bin b finds the pair holding its first tile
// b*budget by binary search over the flat starts, and writes its offset,
// its first descriptor and, when that is not the pair's first, the
// descriptor itself.  Beside its first descriptor each bin also records the
// physical pages of that descriptor's first two tiles, read from the page
// table here, so that the attention kernel's first KV loads follow a single
// round trip.
#include "lbp_internal.h"

namespace lbp {
namespace {

constexpr int kPlanThreads = 1024;
constexpr int kPlanWaves = kPlanThreads / 64;

// Inclusive prefix sum over the 64 lanes of a wave: shifts by 1, 2, 4 and 8
// lanes inside each row of 16 (DPP row_shr), then the gfx9 row broadcasts
// carry row 0 into row 1 and row 2 into row 3 (row_bcast:15), and rows 0-1
// into rows 2-3 (row_bcast:31).  Lanes that a shift or a masked row leaves
// without a source add zero.
__device__ inline int wave_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return x;
}

// Inclusive prefix sum over the 16 lanes of each row.
__device__ inline int row_inclusive_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);
  return x;
}

// Exclusive prefix sums of two values over the block, with one barrier:
// each wave scans its lanes and posts its two totals; after the barrier
// every wave scans the 16 posted totals itself.  tot receives the block
// totals.  lds holds 2 * kPlanWaves ints; a buffer may be posted to again
// only after one more barrier, so consecutive calls alternate two buffers.
__device__ int2 block_exclusive_scan2(int v0, int v1, int* lds, int2* tot) {
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int x0 = wave_inclusive_scan(v0);
  const int x1 = wave_inclusive_scan(v1);
  if (lane == 63) {
    lds[wid] = x0;
    lds[kPlanWaves + wid] = x1;
  }
  __syncthreads();
  int w0 = 0, w1 = 0;
  if (lane < kPlanWaves) {
    w0 = lds[lane];
    w1 = lds[kPlanWaves + lane];
  }
  w0 = row_inclusive_scan(w0);
  w1 = row_inclusive_scan(w1);
  *tot = make_int2(__builtin_amdgcn_readlane(w0, kPlanWaves - 1),
                   __builtin_amdgcn_readlane(w1, kPlanWaves - 1));
  const int b0 = wid ? __builtin_amdgcn_readlane(w0, wid - 1) : 0;
  const int b1 = wid ? __builtin_amdgcn_readlane(w1, wid - 1) : 0;
  return make_int2(b0 + x0 - v0, b1 + x1 - v1);
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

// Per-pair arrays in LDS: the clamped lengths for up to kLenPairs pairs and,
// for up to kArrayPairs pairs, also the flat starts and first descriptor
// slots (so the binary searches read LDS); past those the arrays live in the
// plan workspace and the lengths are re-read from seq_lens.
constexpr int kArrayPairs = 12288;   // 3 x 4 B x 12288 = 144 KB
constexpr int kLenPairs = 36864;     // 4 B x 36864 = 144 KB
constexpr int kLoadBatch = 8;        // length loads a thread keeps in flight

template <bool kLenLds, bool kArraysLds>
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  static_assert(kLenLds || !kArraysLds, "arrays in LDS only with the lengths");
  static_assert(kPlanWaves == 16, "the wave totals are scanned as one DPP row");
  __shared__ int scan_lds[2][2 * kPlanWaves];   // consecutive scans alternate
  extern __shared__ int pair_lds[];   // lengths [npairs], then (kArraysLds) starts, first slots
  const int tid = threadIdx.x;
  const int B = a.batch;
  const int npairs = a.num_kv_heads * B;
  int* const s_len = pair_lds;
  int* const start_of = kArraysLds ? pair_lds + npairs : a.scratch;
  int* const first_of = kArraysLds ? pair_lds + 2 * npairs : a.pair_first;
  // pair p = g*B + r (KV head g, request r) has request r's length; threads
  // walk the pairs in strides of kPlanThreads, carrying (g, r) along
  const int step_g = kPlanThreads / B, step_r = kPlanThreads % B;   // B >= 1 (host check)
  auto advance = [&](int& g, int& r) {
    g += step_g;
    r += step_r;
    if (r >= B) {
      r -= B;
      ++g;
    }
  };

  // clamped lengths (into LDS when they fit), the total tiles T and whether
  // any length was clamped
  int local = 0, clamped = 0;
  {
    int g = tid / B, r = tid % B;
    if constexpr (kLenLds) {
      // up to kLoadBatch coalesced loads in flight per thread (a uniform
      // count; the request index stays in range past the last pair)
      for (int q = 0; q < npairs; q += kLoadBatch * kPlanThreads) {
        const int nb = min(kLoadBatch, (npairs - q + kPlanThreads - 1) / kPlanThreads);
        int L[kLoadBatch];
#pragma unroll
        for (int u = 0; u < kLoadBatch; ++u) {
          if (u < nb) {
            L[u] = a.seq_lens[r];
            advance(g, r);
          }
        }
#pragma unroll
        for (int u = 0; u < kLoadBatch; ++u) {
          const int p = q + u * kPlanThreads + tid;
          if (u < nb && p < npairs) {
            const int Lc = clamp_len(L[u], a.max_tokens, &clamped);
            s_len[p] = Lc;
            local += (Lc + kPageTokens - 1) / kPageTokens;
          }
        }
      }
    } else {
      for (int p = tid; p < npairs; p += kPlanThreads) {
        local += (clamp_len(a.seq_lens[r], a.max_tokens, &clamped) + kPageTokens - 1) / kPageTokens;
        advance(g, r);
      }
    }
  }
  int2 tot;
  block_exclusive_scan2(local, clamped, scan_lds[0], &tot);   // also publishes s_len
  const int T = tot.x;
  const bool any_clamped = tot.y > 0;

  const bool dynamic = a.policy == LBP_POLICY_DYNAMIC;
  const int budget = dynamic ? max((T + a.num_bins - 1) / a.num_bins, a.param) : a.param;
  // descriptors of a pair with n tiles (static plans)
  auto static_count = [&](int n) {
    if (a.policy == LBP_POLICY_STATIC_SPLITS) {
      const int c = (n + budget - 1) / budget;   // ceil(n / S) tiles per split
      return c ? (n + c - 1) / c : 0;
    }
    return (n + budget - 1) / budget;            // ceil(n / C) chunks
  };
  // descriptor j of pair (g, r) with length L and flat start S
  auto desc_of = [&](int g, int r, int L, int S, int j) {
    const int n = (L + kPageTokens - 1) / kPageTokens;
    int lo, hi;
    if (dynamic) {
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
    return make_int4(g, r, lo * kPageTokens, min(hi * kPageTokens, L));
  };
  auto len_at = [&](int p, int r) {
    if constexpr (kLenLds) {
      return s_len[p];
    } else {
      int unused = 0;
      return clamp_len(a.seq_lens[r], a.max_tokens, &unused);
    }
  };

  // rounds of kPlanThreads pairs, one per thread: flat start, first
  // descriptor slot, count, split-list entry and (dynamic plan) the pair's
  // first descriptor
  int carry_s = 0, carry_d = 0, carry_split = 0;
  {
    int g = tid / B, r = tid % B;
    for (int base = 0; base < npairs; base += kPlanThreads) {
      const int p = base + tid;
      const bool valid = p < npairs;
      const int L = valid ? len_at(p, r) : 0;
      const int n = (L + kPageTokens - 1) / kPageTokens;
      int2 t0, t1;
      const int S = carry_s + block_exclusive_scan2(n, 0, scan_lds[1], &t0).x;
      int cnt = 0, hi = 0;
      if (valid && n) {
        if (dynamic) {
          const int bin0 = S / budget;
          const int64_t end0 = int64_t(bin0 + 1) * budget;   // end of the first bin
          cnt = (S + n - 1) / budget - bin0 + 1;
          hi = int(min<int64_t>(S + n, end0) - S);
        } else {
          cnt = static_count(n);
        }
      }
      const int2 ex = block_exclusive_scan2(cnt, cnt >= 2, scan_lds[0], &t1);
      const int first = carry_d + ex.x;
      if (valid) {
        start_of[p] = S;
        first_of[p] = first;
        if constexpr (kArraysLds) a.pair_first[p] = first;
        a.pair_count[p] = cnt;
        const int slot = carry_split + ex.y;
        if (cnt >= 2 && slot < a.max_split)
          reinterpret_cast<int4*>(a.split_list)[slot] = make_int4(p, first, cnt, 0);
        if (dynamic && cnt > 0)
          reinterpret_cast<int4*>(a.desc)[first] = make_int4(g, r, 0, min(hi * kPageTokens, L));
      }
      carry_s += t0.x;
      carry_d += t1.x;
      carry_split += t1.y;
      advance(g, r);
    }
  }
  const int D = carry_d;
  const int nsplit = carry_split;
  __syncthreads();  // the per-pair arrays visible to the block

  // arrival counters of the attention kernel's merge start at zero
  for (int i = tid; i < a.arrive_words; i += kPlanThreads) a.arrive[i] = 0;

  // per bin: its descriptor offset, first descriptor and that descriptor's
  // first two pages (read by the attention kernel together with the range,
  // so its first KV loads need no page-table round trip); in the dynamic
  // plan also the descriptor itself where a bin boundary falls inside a
  // pair, and in the static plans (one descriptor per bin) every descriptor
  int U;
  int4* const bin_first = reinterpret_cast<int4*>(a.bin_first);   // two int4 per bin
  int4* const desc = reinterpret_cast<int4*>(a.desc);
  // pages of descriptor v's first tile and of the next one (its first again
  // for a one-tile descriptor)
  auto first_pages = [&](int r, int4 v) {
    const int32_t* row = a.page_table + int64_t(r) * a.page_table_stride;
    const int t0 = v.z / kPageTokens;
    return make_int4(row[t0], row[min(t0 + 1, (v.w - 1) / kPageTokens)], 0, 0);
  };
  if (dynamic) {
    U = T ? (T + budget - 1) / budget : 0;
    for (int b = tid; b <= a.num_bins; b += kPlanThreads) {
      int off = D;
      int4 v = make_int4(0, 0, 0, 0), pg = v;
      if (b < U) {                   // a used bin holds at least one descriptor
        const int f = b * budget;    // < T, so fits in int
        const int p = last_le(start_of, npairs, f);
        const int S = start_of[p];
        const int j = b - S / budget;
        const int r = p % B;
        off = first_of[p] + j;
        v = desc_of(p / B, r, len_at(p, r), S, j);
        if (j > 0) desc[off] = v;
        pg = first_pages(r, v);
      }
      a.bin_offset[b] = off;
      if (b < a.num_bins) {
        bin_first[2 * b] = v;
        bin_first[2 * b + 1] = pg;
      }
    }
  } else {
    U = D;
    const int Sp = a.splits_per_pair;
    for (int b = tid; b <= a.num_bins; b += kPlanThreads) {
      int off = D;
      int4 v = make_int4(0, 0, 0, 0), pg = v;
      if (b < a.num_bins) {
        const int p = b / Sp, s = b % Sp;
        const int r = p % B;
        const int L = len_at(p, r);
        const int cnt = static_count((L + kPageTokens - 1) / kPageTokens);
        off = first_of[p] + min(s, cnt);
        if (s < cnt) {
          v = desc_of(p / B, r, L, 0, s);
          desc[off] = v;
          pg = first_pages(r, v);
        }
        bin_first[2 * b] = v;
        bin_first[2 * b + 1] = pg;
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
    h[kHdrStatus] = any_clamped ? kStatusClamped : 0;
    for (int i = kHdrStatus + 1; i < kHdrWords; ++i) h[i] = 0;
    h[kHdrSplits] = min(nsplit, a.max_split);
  }
}

}  // namespace

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  PlanArgs copy = a;
  void* args[] = {&copy};
  const int npairs = a.num_kv_heads * a.batch;
  if (npairs <= kArrayPairs)
    return hipLaunchKernel(reinterpret_cast<const void*>(&plan_kernel<true, true>), dim3(1),
                           dim3(kPlanThreads), args, size_t(npairs) * 12, s);
  if (npairs <= kLenPairs)
    return hipLaunchKernel(reinterpret_cast<const void*>(&plan_kernel<true, false>), dim3(1),
                           dim3(kPlanThreads), args, size_t(npairs) * 4, s);
  return hipLaunchKernel(reinterpret_cast<const void*>(&plan_kernel<false, false>), dim3(1),
                         dim3(kPlanThreads), args, 0, s);
}

}  // namespace lbp
