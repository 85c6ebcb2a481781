// LSE combine of split-KV partials into the final BF16 output.
//
// Method (SGLang x HPC-Ops page, "Scheduling around live KV work", second
// paragraph; vLLM x HPC-Ops page, bullet "Compute and combine"): for every
// (KV head, request) pair the combine reads how many partials the task map
// gave it and merges them under the global softmax normalisation:
// with M = max_k lse_k, out = sum_k 2^(lse_k - M) o_k / sum_k 2^(lse_k - M)
// (base-2 log-sum-exp of log2(e)-scaled scores, as the attention kernel
// writes them), rounded to BF16 (nearest even).
//
// gfx950 mapping: one 256-thread workgroup per (pair, query head), so a pair
// split into hundreds of partials (a very long request) is merged by G
// workgroups in parallel rather than one.  Thread t owns dims
// [4(t%32), +4) and partials k = t/32 (mod 8): each partial row of 512 B is
// read fully coalesced, eight partials are in flight per workgroup, and the
// eight online (max, sum, acc) states are merged in LDS in a fixed order, so
// the result is bitwise deterministic.
#include "lbp_internal.h"

namespace lbp {
namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerRow = kHeadDim / 4;         // 32 float4 per 128-dim row
constexpr int kRowsInFlight = kThreads / kLanesPerRow;  // 8

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__global__ __launch_bounds__(kThreads) void combine_kernel(CombineArgs a) {
  __shared__ float red_m[kRowsInFlight];
  __shared__ float red_l[kRowsInFlight];
  __shared__ f32x4_t red_o[kRowsInFlight][kLanesPerRow];

  const int p = blockIdx.x;      // pair = kv_head * batch + request
  const int q = blockIdx.y;      // query head within the group
  const int G = a.group;
  const int g = p / a.batch, r = p % a.batch;
  const int c4 = threadIdx.x % kLanesPerRow;
  const int kg = threadIdx.x / kLanesPerRow;
  const int cnt = a.pair_count[p];
  const int first = a.pair_first[p];

  float m = -INFINITY, l = 0.f;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int k = kg; k < cnt; k += kRowsInFlight) {
    const int64_t slot = int64_t(first + k) * G + q;
    const float lse = a.lse_part[slot];
    const f32x4_t o = reinterpret_cast<const f32x4_t*>(a.o_part + slot * kHeadDim)[c4];
    const float m_new = fmaxf(m, lse);
    const float sa = __builtin_amdgcn_exp2f(m - m_new);
    const float sb = __builtin_amdgcn_exp2f(lse - m_new);
    acc = acc * sa + o * sb;
    l = l * sa + sb;
    m = m_new;
  }
  if (c4 == 0) {
    red_m[kg] = m;
    red_l[kg] = l;
  }
  red_o[kg][c4] = acc;
  __syncthreads();
  if (kg != 0) return;

  f32x4_t out = {0.f, 0.f, 0.f, 0.f};
  if (cnt > 0) {
    float M = -INFINITY;
#pragma unroll
    for (int i = 0; i < kRowsInFlight; ++i) M = fmaxf(M, red_m[i]);
    float L = 0.f;
#pragma unroll
    for (int i = 0; i < kRowsInFlight; ++i) {
      const float c = __builtin_amdgcn_exp2f(red_m[i] - M);
      L += red_l[i] * c;
      out += red_o[i][c4] * c;
    }
    out = out / L;
  }
  bf16x2_t lo = {static_cast<__bf16>(out[0]), static_cast<__bf16>(out[1])};
  bf16x2_t hi = {static_cast<__bf16>(out[2]), static_cast<__bf16>(out[3])};
  uint2 packed = make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
  const int64_t row = int64_t(r) * a.num_q_heads + int64_t(g) * G + q;
  reinterpret_cast<uint2*>(static_cast<char*>(a.out) + row * kHeadDim * 2)[c4] = packed;
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
