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
// gfx950 mapping: one 256-thread workgroup per (pair, query head), so a pair
// split into hundreds of partials (a very long request) is merged by G
// workgroups in parallel.  Pairs with exactly one descriptor were finished
// by the attention kernel and are skipped; pairs with none get zeros.
// Phase 1 loads every log-sum-exp of the pair at once (one per thread) and
// reduces max and weight sum over the block; phase 2 has thread t own dims
// [4(t%32), +4) of partials k = t/32 (mod 8), unrolled four deep so 32
// partial rows are in flight, then merges the eight partial sums in LDS in a
// fixed order (bitwise deterministic).
#include "lbp_internal.h"

namespace lbp {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kLanesPerRow = kHeadDim / 4;              // 32 float4 per 128-dim row
constexpr int kRowGroups = kThreads / kLanesPerRow;     // 8
constexpr int kUnroll = 4;
constexpr int kCachedWeights = 1024;

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}
__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ inline void store_row4(void* out, int64_t row, int c4, f32x4_t v) {
  bf16x2_t lo = {static_cast<__bf16>(v[0]), static_cast<__bf16>(v[1])};
  bf16x2_t hi = {static_cast<__bf16>(v[2]), static_cast<__bf16>(v[3])};
  uint2 packed = make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
  reinterpret_cast<uint2*>(static_cast<char*>(out) + row * kHeadDim * 2)[c4] = packed;
}

__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  __shared__ float red[kWaves];
  __shared__ float weights[kCachedWeights];
  __shared__ f32x4_t part[kRowGroups][kLanesPerRow];

  const int p = blockIdx.x;      // pair = kv_head * batch + request
  const int q = blockIdx.y;      // query head within the group
  const int cnt = a.pair_count[p];
  if (cnt == 1) return;          // finished in place by the attention kernel
  const int G = a.group;
  const int g = p / a.batch, r = p % a.batch;
  const int64_t row = int64_t(r) * a.num_q_heads + int64_t(g) * G + q;
  const int t = threadIdx.x;
  const int c4 = t % kLanesPerRow;
  const int kg = t / kLanesPerRow;
  if (cnt == 0) {                // no tokens: zero output
    if (kg == 0) store_row4(a.out, row, c4, f32x4_t{0.f, 0.f, 0.f, 0.f});
    return;
  }
  const int first = a.pair_first[p];
  const float* lse = a.lse_part + int64_t(first) * G + q;

  // phase 1: M = max lse, S = sum 2^(lse - M)
  float mx = -INFINITY;
  for (int k = t; k < cnt; k += kThreads) mx = fmaxf(mx, lse[int64_t(k) * G]);
  mx = wave_max(mx);
  if ((t & 63) == 0) red[t >> 6] = mx;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) M = fmaxf(M, red[w]);
  __syncthreads();
  float sum = 0.f;
  for (int k = t; k < cnt; k += kThreads) {
    const float w = __builtin_amdgcn_exp2f(lse[int64_t(k) * G] - M);
    if (k < kCachedWeights) weights[k] = w;
    sum += w;
  }
  sum = wave_sum(sum);
  if ((t & 63) == 0) red[t >> 6] = sum;
  __syncthreads();
  float S = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) S += red[w];

  // phase 2: weighted sum of the partial rows
  const f32x4_t* o = reinterpret_cast<const f32x4_t*>(a.o_part + (int64_t(first) * G + q) * kHeadDim);
  const int64_t stride4 = int64_t(G) * kLanesPerRow;   // float4s between consecutive partials
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  int k = kg;
  for (; k + (kUnroll - 1) * kRowGroups < cnt; k += kUnroll * kRowGroups) {
    f32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = o[int64_t(k + u * kRowGroups) * stride4 + c4];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int kk = k + u * kRowGroups;
      const float w = kk < kCachedWeights ? weights[kk]
                                          : __builtin_amdgcn_exp2f(lse[int64_t(kk) * G] - M);
      acc += v[u] * w;
    }
  }
  for (; k < cnt; k += kRowGroups) {
    const float w = k < kCachedWeights ? weights[k]
                                       : __builtin_amdgcn_exp2f(lse[int64_t(k) * G] - M);
    acc += o[int64_t(k) * stride4 + c4] * w;
  }
  part[kg][c4] = acc;
  __syncthreads();
  if (kg != 0) return;
  f32x4_t tot = part[0][c4];
#pragma unroll
  for (int i = 1; i < kRowGroups; ++i) tot += part[i][c4];
  store_row4(a.out, row, c4, tot / S);
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, int npairs, hipStream_t s) {
  if (npairs <= 0) return hipSuccess;
  CombineArgs copy = a;
  void* args[] = {&copy};
  return hipLaunchKernel(reinterpret_cast<const void*>(&combine_kernel), dim3(npairs, a.group),
                         dim3(kThreads), args, 0, s);
}

}  // namespace lbp
