// Fused attention prologue for the new tokens of one decode step.
//
// Method (SGLang x HPC-Ops page, "A fused attention prologue"; vLLM x
// HPC-Ops page, the HpcRopeNorm paragraph of the Attention backend
// section): straight from the fused QKV projection, QK-Norm (RMSNorm over
// each head's 128 dims with a learned weight) is applied to every query and
// key head before RoPE, K and V are written directly into the paged cache at
// the new token's slot, and with an FP8 query the query leaves in e4m3 with
// one scale per (token, head), ready for the attention kernel without
// requantization.  RoPE rotates dim pairs (i, i + 64) by the angles of the
// token's position, read from a caller-supplied cos/sin table.  The q_len
// new tokens of request r (one for plain decode, more for speculative
// verification) sit at positions seq_lens[r] - q_len + j.
//
// gfx950 mapping: the step is a few KB per request and bound by memory
// latency, not arithmetic, so there is no MFMA.  One wave handles one
// (request, token, head) row of 128 dims: lane l owns dims l and l + 64, which is
// exactly one RoPE pair, so the rotation needs no cross-lane exchange; the
// RMSNorm sum of squares and the FP8 row maximum are wave reductions.  Four
// rows per 256-thread workgroup.  FP8 rows: scale = max |x| / 448 (1 for an
// all-zero row), code = e4m3 nearest to x * (448 / max |x|) after clamping to
// +-448.
#include "lbp_internal.h"

namespace lbp {
namespace {

constexpr int kRowsPerBlock = 4;
constexpr float kE4m3Max = 448.f;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}
__device__ inline float wave_max(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

__device__ inline float bf16_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, uint32_t(b) << 16);
}

// e4m3 code of x (|x| <= 448 after the clamp), nearest value, ties to even.
__device__ inline uint8_t e4m3_code(float x) {
  x = fminf(fmaxf(x, -kE4m3Max), kE4m3Max);
  const int packed = __builtin_amdgcn_cvt_pk_fp8_f32(x, 0.f, 0, false);
  return uint8_t(packed & 0xFF);
}

// Per-row FP8: returns this lane's two codes and (wave-uniform) the row scale.
__device__ inline void quantize_pair(float z0, float z1, uint8_t& c0, uint8_t& c1,
                                     float& scale) {
  const float amax = wave_max(fmaxf(fabsf(z0), fabsf(z1)));
  const bool zero = !(amax > 0.f);
  scale = zero ? 1.f : amax / kE4m3Max;
  const float inv = zero ? 1.f : kE4m3Max / amax;
  c0 = e4m3_code(z0 * inv);
  c1 = e4m3_code(z1 * inv);
}

__global__ __launch_bounds__(kRowsPerBlock * 64) void prologue_kernel(PrologueArgs a) {
  const int H3 = a.num_q_heads + 2 * a.num_kv_heads;
  const int row = blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= a.batch * a.q_len * H3) return;   // whole wave
  const int lane = threadIdx.x & 63;
  const int rt = row / H3, h = row % H3;        // rt = request * q_len + token
  const int r = rt / a.q_len, j = rt % a.q_len;
  const int L = a.seq_lens[r];
  const int pos = L - a.q_len + j;   // new token j of request r
  if (pos < 0) return;               // before the sequence start: no token
  const int prow = min(pos, a.max_position - 1);

  const uint16_t* x = static_cast<const uint16_t*>(a.qkv) + (int64_t(rt) * H3 + h) * kHeadDim;
  float z0 = bf16_to_f32(x[lane]);
  float z1 = bf16_to_f32(x[lane + 64]);
  const bool is_q = h < a.num_q_heads;
  const bool is_v = h >= a.num_q_heads + a.num_kv_heads;
  if (!is_v) {
    // QK-Norm, then RoPE on the pair (lane, lane + 64)
    const float ms = wave_sum(z0 * z0 + z1 * z1) * (1.f / kHeadDim);
    const float inv_rms = 1.f / sqrtf(ms + a.norm_eps);
    const float* w = is_q ? a.q_norm_weight : a.k_norm_weight;
    const float y0 = z0 * inv_rms * w[lane];
    const float y1 = z1 * inv_rms * w[lane + 64];
    const float* cs = a.rope_cos_sin + int64_t(prow) * kHeadDim;
    const float c = cs[lane], s = cs[64 + lane];
    z0 = y0 * c - y1 * s;
    z1 = y1 * c + y0 * s;
  }

  if (is_q) {
    const int64_t qrow = int64_t(rt) * a.num_q_heads + h;
    if (a.q_fp8) {
      uint8_t c0, c1;
      float scale;
      quantize_pair(z0, z1, c0, c1, scale);
      uint8_t* qo = static_cast<uint8_t*>(a.q_out) + qrow * kHeadDim;
      qo[lane] = c0;
      qo[lane + 64] = c1;
      if (lane == 0) a.q_scale_out[qrow] = scale;
    } else {
      __bf16* qo = static_cast<__bf16*>(a.q_out) + qrow * kHeadDim;
      qo[lane] = static_cast<__bf16>(z0);
      qo[lane + 64] = static_cast<__bf16>(z1);
    }
    return;
  }

  // K or V of KV head hk into the new token's slot
  if (pos >= a.max_tokens) return;   // past the page table's capacity
  const int hk = is_v ? h - a.num_q_heads - a.num_kv_heads : h - a.num_q_heads;
  const int page = a.page_table[int64_t(r) * a.page_table_stride + (pos >> 6)];
  const int64_t slot = (int64_t(page) * a.num_kv_heads + hk) * kPageTokens + (pos & 63);
  void* cache = is_v ? a.v_cache : a.k_cache;
  if (a.kv_fp8) {
    uint8_t c0, c1;
    float scale;
    quantize_pair(z0, z1, c0, c1, scale);
    uint8_t* dst = static_cast<uint8_t*>(cache) + slot * kHeadDim;
    dst[lane] = c0;
    dst[lane + 64] = c1;
    if (lane == 0) (is_v ? a.v_scale : a.k_scale)[slot] = scale;
  } else {
    __bf16* dst = static_cast<__bf16*>(cache) + slot * kHeadDim;
    dst[lane] = static_cast<__bf16>(z0);
    dst[lane + 64] = static_cast<__bf16>(z1);
  }
}

}  // namespace

hipError_t launch_prologue(const PrologueArgs& a, hipStream_t s) {
  const int rows = a.batch * a.q_len * (a.num_q_heads + 2 * a.num_kv_heads);
  if (rows <= 0) return hipSuccess;
  PrologueArgs copy = a;
  void* args[] = {&copy};
  return hipLaunchKernel(reinterpret_cast<const void*>(&prologue_kernel),
                         dim3((rows + kRowsPerBlock - 1) / kRowsPerBlock), dim3(kRowsPerBlock * 64),
                         args, 0, s);
}

}  // namespace lbp
