// Log-sum-exp merge of normalised partial outputs, shared by the combine
// kernel and the merge the attention kernel performs for split pairs.
//
// Method (SGLang x HPC-Ops page, "Scheduling around live KV work", second
// paragraph; vLLM x HPC-Ops page, bullet "Compute and combine"): partials
// (o_k, lse_k) of one query row, each normalised over its own token range,
// merge under the global softmax normalisation as
// out = sum_k 2^(lse_k - M) o_k / sum_k 2^(lse_k - M), M = max_k lse_k.
// The log-sum-exps are base 2 over log2(e)-scaled scores, as the attention
// kernel writes them.
#pragma once

#include "lbp_internal.h"

namespace lbp {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// x if finite, else 0: the reference point of an exponent when every term
// is -inf (an empty state), so that exp2(-inf - ref) = 0 instead of NaN.
__device__ inline float finite_or_zero(float x) { return x == -INFINITY ? 0.f : x; }

// Online merge of one more (lse, row) into a running (max, sum, acc) state;
// an empty state (and an empty partial) has m = -inf, l = 0, acc = 0.
__device__ inline void merge_into(float& m, float& l, f32x4_t& acc, float lse, f32x4_t o) {
  const float m_new = fmaxf(m, lse);
  const float ref = finite_or_zero(m_new);
  const float a = __builtin_amdgcn_exp2f(m - ref);     // 0 while the state is empty
  const float b = __builtin_amdgcn_exp2f(lse - ref);   // 0 for an empty partial
  acc = acc * a + o * b;
  l = l * a + b;
  m = m_new;
}

// Four consecutive dims [4*c4, 4*c4 + 4) of output row `row`, rounded to
// BF16 (nearest even) and stored as one 8-byte write.
__device__ inline void store_bf16x4(void* out, int64_t row, int c4, f32x4_t v) {
  bf16x2_t lo = {static_cast<__bf16>(v[0]), static_cast<__bf16>(v[1])};
  bf16x2_t hi = {static_cast<__bf16>(v[2]), static_cast<__bf16>(v[3])};
  uint2 packed = make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
  reinterpret_cast<uint2*>(static_cast<char*>(out) + row * kHeadDim * 2)[c4] = packed;
}

}  // namespace lbp
